// Host packer: canonical Q8G64 / Q4G32 weights -> the streaming layout in
// layout.h, and back.  Runs once per weight matrix, on the host; the caller
// uploads the result.  Fixing the layout once at load time, keeping every
// row K-contiguous within its group, and permuting only whole row-groups
// follows the observations that row permutation is safe for block formats
// while column permutation crosses groups (vllm.cpp pull request #1936,
// "perf(GFX1100-TG200)" commit log) and that the decode GEMV should read the
// quantized bytes directly in wide contiguous loads (zLLM GLM-5.3 ROCm
// decode post, "W8 direct read" section and bottleneck table).
#include <string.h>

#include "../../include/qgemv.h"
#include "layout.h"

namespace {

// Row of (tile, r, rho).
inline int64_t row_of(const qg::Layout& L, int64_t t, int r, int rho)
{
    return t * L.TR + int64_t(r) * (64 / L.G) + rho;
}

// Q4 unit: 32 canonical codes (16 bytes, even k in the low nibble) -> 4
// dwords where dword d holds k = 8d..8d+7 with k = 8d+2p in bits 4p..4p+3
// and k = 8d+2p+1 in bits 16+4p..19+4p.  Masking (dword >> 4p) & 0x000F000F
// then yields the codes of the bf16 activation pair (x[8d+2p], x[8d+2p+1]).
inline void q4_unit_pack(const uint8_t* src16, uint8_t* dst16)
{
    uint8_t c[32];
    for (int b = 0; b < 16; ++b) {
        c[2 * b] = src16[b] & 0x0f;
        c[2 * b + 1] = src16[b] >> 4;
    }
    for (int d = 0; d < 4; ++d) {
        uint32_t v = 0;
        for (int p = 0; p < 4; ++p) {
            v |= uint32_t(c[8 * d + 2 * p]) << (4 * p);
            v |= uint32_t(c[8 * d + 2 * p + 1]) << (16 + 4 * p);
        }
        memcpy(dst16 + 4 * d, &v, 4);
    }
}

inline void q4_unit_unpack(const uint8_t* src16, uint8_t* dst16)
{
    uint8_t c[32];
    for (int d = 0; d < 4; ++d) {
        uint32_t v;
        memcpy(&v, src16 + 4 * d, 4);
        for (int p = 0; p < 4; ++p) {
            c[8 * d + 2 * p] = (v >> (4 * p)) & 0x0f;
            c[8 * d + 2 * p + 1] = (v >> (16 + 4 * p)) & 0x0f;
        }
    }
    for (int b = 0; b < 16; ++b) dst16[b] = uint8_t(c[2 * b] | (c[2 * b + 1] << 4));
}

// Byte offsets inside the packed buffer.
inline int64_t code_off(const qg::Layout& L, int64_t t, int64_t j, int r, int lane)
{
    return ((t * L.J + j) * L.R + r) * 1024 + int64_t(lane) * 16;
}

// Start of the meta of (tile t, step j).
inline int64_t meta_base(const qg::Layout& L, int64_t t, int64_t j)
{
    return L.code_bytes + t * (L.J * L.meta_step_bytes + L.meta_tile_bytes) + j * L.meta_step_bytes;
}

// Grouped 8-bit formats: lanes_per_group lanes (4 for Q8G64, 8 for Q8G128)
// share one fp16 scale per row slot.
inline int64_t meta_off_q8(const qg::Layout& L, int64_t t, int64_t j, int r, int rho, int a,
                           int lanes_per_group)
{
    return meta_base(L, t, j) + ((int64_t(rho) * (L.G / lanes_per_group) + a) * L.R + r) * 2;
}

inline int64_t meta_off_q4(const qg::Layout& L, int64_t t, int64_t j, int r, int lane)
{
    return meta_base(L, t, j) + (int64_t(lane) * L.R + r) * 4;
}

// Q8PC: the tile's row scales follow its steps' (empty) meta, ordered [rho][r].
inline int64_t meta_off_pc(const qg::Layout& L, int64_t t, int r, int rho)
{
    return meta_base(L, t, L.J) + (int64_t(rho) * L.R + r) * 4;
}

// Packs any 8-bit-code format: the signed codes as they are, then the format's scales.
// scales: fp16 [N][K/group] for the grouped formats, fp32 bit patterns [N] for Q8PC.
qg_status pack_q8(int fmt, const int8_t* q, const void* scales, int64_t N, int64_t K, void* out,
                  size_t out_bytes)
{
    qg::Layout L;
    if (!q || !scales || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(fmt, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    uint8_t* o = static_cast<uint8_t*>(out);
    // Padding rows: code 0, scale 0.
    memset(o, 0, size_t(L.total_bytes));
    const int lanes_per_group = fmt == qg::FMT_Q8G128 ? 8 : 4;
    const int64_t groups = K / L.group;
    const uint16_t* s16 = static_cast<const uint16_t*>(scales);
    const uint32_t* s32 = static_cast<const uint32_t*>(scales);
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    const int64_t n = row_of(L, t, r, rho);
                    if (n >= N) continue;
                    const int64_t u = j * L.G + g;
                    const int8_t* src = q + n * K + u * 16;
                    uint8_t* dst = o + code_off(L, t, j, r, lane);
                    memcpy(dst, src, 16);
                    if (fmt == qg::FMT_Q8PC) {
                        if (j == 0 && g == 0) memcpy(o + meta_off_pc(L, t, r, rho), &s32[n], 4);
                    } else if (g % lanes_per_group == 0) {
                        const uint16_t sv = s16[n * groups + (u * 16) / L.group];
                        memcpy(o + meta_off_q8(L, t, j, r, rho, g / lanes_per_group, lanes_per_group),
                               &sv, 2);
                    }
                }
    return QG_OK;
}

qg_status unpack_q8(int fmt, const void* packed, size_t packed_bytes, int64_t N, int64_t K, int8_t* q,
                    void* scales)
{
    qg::Layout L;
    if (!packed || !q || !scales) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(fmt, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    const int lanes_per_group = fmt == qg::FMT_Q8G128 ? 8 : 4;
    const int64_t groups = K / L.group;
    uint16_t* s16 = static_cast<uint16_t*>(scales);
    uint32_t* s32 = static_cast<uint32_t*>(scales);
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    const int64_t n = row_of(L, t, r, rho);
                    if (n >= N) continue;
                    const int64_t u = j * L.G + g;
                    const uint8_t* src = p + code_off(L, t, j, r, lane);
                    memcpy(q + n * K + u * 16, src, 16);
                    if (fmt == qg::FMT_Q8PC) {
                        if (j == 0 && g == 0) memcpy(&s32[n], p + meta_off_pc(L, t, r, rho), 4);
                    } else if (g % lanes_per_group == 0) {
                        memcpy(&s16[n * groups + (u * 16) / L.group],
                               p + meta_off_q8(L, t, j, r, rho, g / lanes_per_group, lanes_per_group), 2);
                    }
                }
    return QG_OK;
}

// A canonical Q4G32 matrix (codes [N][K/2], scale and min [N][K/32]).  The
// pointers are writable only for unpacking.
struct Q4Rows {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* mins;
};

// Packs the rows of layout L; source(n, &row) names the canonical matrix and
// row that packed row n comes from, or returns null for a padding row (code
// 0, scale 0, min 0).
template <class Source>
void pack_q4(const qg::Layout& L, int64_t K, Source source, void* out)
{
    uint8_t* o = static_cast<uint8_t*>(out);
    memset(o, 0, size_t(L.total_bytes));
    const int64_t groups = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    int64_t n;
                    const Q4Rows* m = source(row_of(L, t, r, rho), &n);
                    if (!m) continue;
                    const int64_t u = j * L.G + g;
                    q4_unit_pack(m->codes + n * (K / 2) + u * 16, o + code_off(L, t, j, r, lane));
                    const uint32_t meta = uint32_t(m->scales[n * groups + u]) |
                                          (uint32_t(m->mins[n * groups + u]) << 16);
                    memcpy(o + meta_off_q4(L, t, j, r, lane), &meta, 4);
                }
}

template <class Source>
void unpack_q4(const qg::Layout& L, int64_t K, Source source, const void* packed)
{
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    const int64_t groups = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    int64_t n;
                    const Q4Rows* m = source(row_of(L, t, r, rho), &n);
                    if (!m) continue;
                    const int64_t u = j * L.G + g;
                    q4_unit_unpack(p + code_off(L, t, j, r, lane),
                                   const_cast<uint8_t*>(m->codes) + n * (K / 2) + u * 16);
                    uint32_t meta;
                    memcpy(&meta, p + meta_off_q4(L, t, j, r, lane), 4);
                    const_cast<uint16_t*>(m->scales)[n * groups + u] = uint16_t(meta & 0xffff);
                    const_cast<uint16_t*>(m->mins)[n * groups + u] = uint16_t(meta >> 16);
                }
}

// Gate/up pair layout (layout.h): packed row v of tile t = v / (2 rps) is
// gate row t*rps + (v mod rps) in the first rps rows of the tile and the up
// row with that index in the next rps.
inline const Q4Rows* gate_up_source(int64_t v, int64_t N, int64_t rps, const Q4Rows& gate,
                                    const Q4Rows& up, int64_t* row)
{
    const int64_t t = v / (2 * rps), w = v % (2 * rps);
    *row = t * rps + w % rps;
    if (*row >= N) return nullptr;
    return w < rps ? &gate : &up;
}

// Matrix-core layout (layout.h, MmaLayout): pack / unpack any 8-bit format.
// scales: fp16 [N][K/group] (Q8G64, Q8G128) or fp32 bit patterns [N] (Q8PC).
qg_status pack_q8_mma(int fmt, const int8_t* q, const void* scales, int64_t N, int64_t K, void* out,
                      size_t out_bytes)
{
    qg::MmaLayout L;
    if (!q || !scales || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_mma_layout(fmt, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    uint8_t* o = static_cast<uint8_t*>(out);
    memset(o, 0, size_t(L.total_bytes));   // padding rows: code 0, scale 0
    const uint16_t* s16 = static_cast<const uint16_t*>(scales);
    const uint32_t* s32 = static_cast<const uint32_t*>(scales);
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int rho = 0; rho < qg::kMmaRows; ++rho) {
            const int64_t n = t * qg::kMmaRows + rho;
            if (n >= N) continue;
            for (int64_t j = 0; j < L.J; ++j)
                for (int qs = 0; qs < 4; ++qs) {
                    const int lane = qs * 16 + rho;
                    const int8_t* src = q + n * K + 64 * j + 16 * qs;
                    uint8_t* dst = o + (t * L.J + j) * 1024 + lane * 16;
                    memcpy(dst, src, 16);
                }
            uint8_t* meta = o + L.code_bytes + t * L.meta_tile_bytes;
            if (fmt == qg::FMT_Q8PC) {
                memcpy(meta + rho * 4, &s32[n], 4);
            } else {
                for (int64_t g = 0; g < L.groups; ++g)
                    memcpy(meta + (g * qg::kMmaRows + rho) * 2, &s16[n * L.groups + g], 2);
            }
        }
    return QG_OK;
}

qg_status unpack_q8_mma(int fmt, const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                        int8_t* q, void* scales)
{
    qg::MmaLayout L;
    if (!packed || !q || !scales) return QG_ERR_INVALID_ARG;
    if (!qg::make_mma_layout(fmt, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    uint16_t* s16 = static_cast<uint16_t*>(scales);
    uint32_t* s32 = static_cast<uint32_t*>(scales);
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int rho = 0; rho < qg::kMmaRows; ++rho) {
            const int64_t n = t * qg::kMmaRows + rho;
            if (n >= N) continue;
            for (int64_t j = 0; j < L.J; ++j)
                for (int qs = 0; qs < 4; ++qs) {
                    const uint8_t* src = p + (t * L.J + j) * 1024 + (qs * 16 + rho) * 16;
                    memcpy(q + n * K + 64 * j + 16 * qs, src, 16);
                }
            const uint8_t* meta = p + L.code_bytes + t * L.meta_tile_bytes;
            if (fmt == qg::FMT_Q8PC) {
                memcpy(&s32[n], meta + rho * 4, 4);
            } else {
                for (int64_t g = 0; g < L.groups; ++g)
                    memcpy(&s16[n * L.groups + g], meta + (g * qg::kMmaRows + rho) * 2, 2);
            }
        }
    return QG_OK;
}

// Q4G32 in the matrix-core layout (layout.h): codes [N][K/2] canonical
// (even k in the low nibble), scale and min fp16 [N][K/32].  Dword g of
// lane (qs, rho) is the four canonical bytes of row rho's codes at
// k = 128 j + 32 g + 8 qs .. + 7.
qg_status pack_q4_mma(const uint8_t* codes, const uint16_t* scale, const uint16_t* minv, int64_t N,
                      int64_t K, void* out, size_t out_bytes)
{
    qg::MmaLayout L;
    if (!codes || !scale || !minv || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_mma_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    uint8_t* o = static_cast<uint8_t*>(out);
    memset(o, 0, size_t(L.total_bytes));
    const int64_t G = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int rho = 0; rho < qg::kMmaRows; ++rho) {
            const int64_t n = t * qg::kMmaRows + rho;
            if (n >= N) continue;
            for (int64_t j = 0; j < L.J; ++j) {
                for (int qs = 0; qs < 4; ++qs) {
                    uint8_t* dst = o + (t * L.J + j) * 1024 + (qs * 16 + rho) * 16;
                    for (int g = 0; g < 4; ++g)
                        memcpy(dst + 4 * g, codes + n * (K / 2) + (128 * j + 32 * g + 8 * qs) / 2, 4);
                }
                uint8_t* meta = o + L.code_bytes + t * L.meta_tile_bytes + (j * qg::kMmaRows + rho) * 16;
                for (int g = 0; g < 4; ++g) {
                    const int64_t gi = n * G + 4 * j + g;
                    memcpy(meta + 4 * g, &scale[gi], 2);
                    memcpy(meta + 4 * g + 2, &minv[gi], 2);
                }
            }
        }
    return QG_OK;
}

qg_status unpack_q4_mma(const void* packed, size_t packed_bytes, int64_t N, int64_t K, uint8_t* codes,
                        uint16_t* scale, uint16_t* minv)
{
    qg::MmaLayout L;
    if (!packed || !codes || !scale || !minv) return QG_ERR_INVALID_ARG;
    if (!qg::make_mma_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    const int64_t G = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int rho = 0; rho < qg::kMmaRows; ++rho) {
            const int64_t n = t * qg::kMmaRows + rho;
            if (n >= N) continue;
            for (int64_t j = 0; j < L.J; ++j) {
                for (int qs = 0; qs < 4; ++qs) {
                    const uint8_t* src = p + (t * L.J + j) * 1024 + (qs * 16 + rho) * 16;
                    for (int g = 0; g < 4; ++g)
                        memcpy(codes + n * (K / 2) + (128 * j + 32 * g + 8 * qs) / 2, src + 4 * g, 4);
                }
                const uint8_t* meta = p + L.code_bytes + t * L.meta_tile_bytes + (j * qg::kMmaRows + rho) * 16;
                for (int g = 0; g < 4; ++g) {
                    const int64_t gi = n * G + 4 * j + g;
                    memcpy(&scale[gi], meta + 4 * g, 2);
                    memcpy(&minv[gi], meta + 4 * g + 2, 2);
                }
            }
        }
    return QG_OK;
}

}  // namespace

extern "C" {

size_t qpack_q8g64_size(int64_t N, int64_t K)
{
    qg::Layout L;
    return qg::make_layout(qg::FMT_Q8G64, N, K, &L) ? size_t(L.total_bytes) : 0;
}

size_t qpack_q4g32_size(int64_t N, int64_t K)
{
    qg::Layout L;
    return qg::make_layout(qg::FMT_Q4G32, N, K, &L) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q8g64(const int8_t* q, const uint16_t* scales_f16, int64_t N, int64_t K,
                      void* out, size_t out_bytes)
{
    return pack_q8(qg::FMT_Q8G64, q, scales_f16, N, K, out, out_bytes);
}

qg_status qunpack_q8g64(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                        int8_t* q, uint16_t* scales_f16)
{
    return unpack_q8(qg::FMT_Q8G64, packed, packed_bytes, N, K, q, scales_f16);
}

size_t qpack_q8g128_size(int64_t N, int64_t K)
{
    qg::Layout L;
    return qg::make_layout(qg::FMT_Q8G128, N, K, &L) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q8g128(const int8_t* q, const uint16_t* scales_f16, int64_t N, int64_t K,
                       void* out, size_t out_bytes)
{
    return pack_q8(qg::FMT_Q8G128, q, scales_f16, N, K, out, out_bytes);
}

qg_status qunpack_q8g128(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                         int8_t* q, uint16_t* scales_f16)
{
    return unpack_q8(qg::FMT_Q8G128, packed, packed_bytes, N, K, q, scales_f16);
}

size_t qpack_q8pc_size(int64_t N, int64_t K)
{
    qg::Layout L;
    return qg::make_layout(qg::FMT_Q8PC, N, K, &L) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q8pc(const int8_t* q, const float* scales_f32, int64_t N, int64_t K, void* out,
                     size_t out_bytes)
{
    return pack_q8(qg::FMT_Q8PC, q, scales_f32, N, K, out, out_bytes);
}

qg_status qunpack_q8pc(const void* packed, size_t packed_bytes, int64_t N, int64_t K, int8_t* q,
                       float* scales_f32)
{
    return unpack_q8(qg::FMT_Q8PC, packed, packed_bytes, N, K, q, scales_f32);
}

qg_status qpack_q4g32(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* mins_f16,
                      int64_t N, int64_t K, void* out, size_t out_bytes)
{
    qg::Layout L;
    if (!codes || !scales_f16 || !mins_f16 || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const Q4Rows m{codes, scales_f16, mins_f16};
    pack_q4(L, K, [&](int64_t n, int64_t* row) { *row = n; return n < N ? &m : nullptr; }, out);
    return QG_OK;
}

qg_status qunpack_q4g32(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                        uint8_t* codes, uint16_t* scales_f16, uint16_t* mins_f16)
{
    qg::Layout L;
    if (!packed || !codes || !scales_f16 || !mins_f16) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const Q4Rows m{codes, scales_f16, mins_f16};
    unpack_q4(L, K, [&](int64_t n, int64_t* row) { *row = n; return n < N ? &m : nullptr; }, packed);
    return QG_OK;
}

size_t qpack_q8g64_mma_size(int64_t N, int64_t K)
{
    qg::MmaLayout L;
    return qg::make_mma_layout(qg::FMT_Q8G64, N, K, &L) ? size_t(L.total_bytes) : 0;
}

size_t qpack_q8g128_mma_size(int64_t N, int64_t K)
{
    qg::MmaLayout L;
    return qg::make_mma_layout(qg::FMT_Q8G128, N, K, &L) ? size_t(L.total_bytes) : 0;
}

size_t qpack_q8pc_mma_size(int64_t N, int64_t K)
{
    qg::MmaLayout L;
    return qg::make_mma_layout(qg::FMT_Q8PC, N, K, &L) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q8g64_mma(const int8_t* q, const uint16_t* scales_f16, int64_t N, int64_t K,
                          void* out, size_t out_bytes)
{
    return pack_q8_mma(qg::FMT_Q8G64, q, scales_f16, N, K, out, out_bytes);
}

qg_status qpack_q8g128_mma(const int8_t* q, const uint16_t* scales_f16, int64_t N, int64_t K,
                           void* out, size_t out_bytes)
{
    return pack_q8_mma(qg::FMT_Q8G128, q, scales_f16, N, K, out, out_bytes);
}

qg_status qpack_q8pc_mma(const int8_t* q, const float* scales_f32, int64_t N, int64_t K, void* out,
                         size_t out_bytes)
{
    return pack_q8_mma(qg::FMT_Q8PC, q, scales_f32, N, K, out, out_bytes);
}

size_t qpack_q4g32_mma_size(int64_t N, int64_t K)
{
    qg::MmaLayout L;
    return qg::make_mma_layout(qg::FMT_Q4G32, N, K, &L) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q4g32_mma(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* mins_f16,
                          int64_t N, int64_t K, void* out, size_t out_bytes)
{
    return pack_q4_mma(codes, scales_f16, mins_f16, N, K, out, out_bytes);
}

qg_status qunpack_q4g32_mma(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                            uint8_t* codes, uint16_t* scales_f16, uint16_t* mins_f16)
{
    return unpack_q4_mma(packed, packed_bytes, N, K, codes, scales_f16, mins_f16);
}

qg_status qunpack_q8g64_mma(const void* packed, size_t packed_bytes, int64_t N, int64_t K, int8_t* q,
                            uint16_t* scales_f16)
{
    return unpack_q8_mma(qg::FMT_Q8G64, packed, packed_bytes, N, K, q, scales_f16);
}

qg_status qunpack_q8g128_mma(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                             int8_t* q, uint16_t* scales_f16)
{
    return unpack_q8_mma(qg::FMT_Q8G128, packed, packed_bytes, N, K, q, scales_f16);
}

qg_status qunpack_q8pc_mma(const void* packed, size_t packed_bytes, int64_t N, int64_t K, int8_t* q,
                           float* scales_f32)
{
    return unpack_q8_mma(qg::FMT_Q8PC, packed, packed_bytes, N, K, q, scales_f32);
}

size_t qpack_q4g32_gate_up_size(int64_t N, int64_t K)
{
    qg::Layout L;
    int64_t rps;
    return qg::make_gate_up_layout(N, K, &L, &rps) ? size_t(L.total_bytes) : 0;
}

qg_status qpack_q4g32_gate_up(const uint8_t* gate_codes, const uint16_t* gate_scales_f16,
                              const uint16_t* gate_mins_f16, const uint8_t* up_codes,
                              const uint16_t* up_scales_f16, const uint16_t* up_mins_f16,
                              int64_t N, int64_t K, void* out, size_t out_bytes)
{
    qg::Layout L;
    int64_t rps;
    if (!gate_codes || !gate_scales_f16 || !gate_mins_f16 || !up_codes || !up_scales_f16 ||
        !up_mins_f16 || !out)
        return QG_ERR_INVALID_ARG;
    if (!qg::make_gate_up_layout(N, K, &L, &rps)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const Q4Rows gate{gate_codes, gate_scales_f16, gate_mins_f16};
    const Q4Rows up{up_codes, up_scales_f16, up_mins_f16};
    pack_q4(L, K, [&](int64_t v, int64_t* row) { return gate_up_source(v, N, rps, gate, up, row); },
            out);
    return QG_OK;
}

qg_status qunpack_q4g32_gate_up(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                                uint8_t* gate_codes, uint16_t* gate_scales_f16,
                                uint16_t* gate_mins_f16, uint8_t* up_codes,
                                uint16_t* up_scales_f16, uint16_t* up_mins_f16)
{
    qg::Layout L;
    int64_t rps;
    if (!packed || !gate_codes || !gate_scales_f16 || !gate_mins_f16 || !up_codes ||
        !up_scales_f16 || !up_mins_f16)
        return QG_ERR_INVALID_ARG;
    if (!qg::make_gate_up_layout(N, K, &L, &rps)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const Q4Rows gate{gate_codes, gate_scales_f16, gate_mins_f16};
    const Q4Rows up{up_codes, up_scales_f16, up_mins_f16};
    unpack_q4(L, K, [&](int64_t v, int64_t* row) { return gate_up_source(v, N, rps, gate, up, row); },
              packed);
    return QG_OK;
}

}  // extern "C"
