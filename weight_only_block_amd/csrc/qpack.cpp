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

inline int64_t meta_off_q8(const qg::Layout& L, int64_t t, int64_t j, int r, int rho, int a)
{
    return L.code_bytes + (t * L.J + j) * L.meta_step_bytes +
           ((int64_t(rho) * (L.G / 4) + a) * L.R + r) * 2;
}

inline int64_t meta_off_q4(const qg::Layout& L, int64_t t, int64_t j, int r, int lane)
{
    return L.code_bytes + (t * L.J + j) * L.meta_step_bytes + (int64_t(lane) * L.R + r) * 4;
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
    qg::Layout L;
    if (!q || !scales_f16 || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q8G64, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    uint8_t* o = static_cast<uint8_t*>(out);
    // Padding rows: code byte 0x80 (q = 0 after the +128 bias), scale 0.
    memset(o, 0x80, size_t(L.code_bytes));
    memset(o + L.code_bytes, 0, size_t(L.total_bytes - L.code_bytes));
    const int64_t groups = K / 64;
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
                    for (int b = 0; b < 16; ++b) dst[b] = uint8_t(int(src[b]) + 128);
                    if (g % 4 == 0) {
                        const uint16_t s = scales_f16[n * groups + u / 4];
                        memcpy(o + meta_off_q8(L, t, j, r, rho, g / 4), &s, 2);
                    }
                }
    return QG_OK;
}

qg_status qunpack_q8g64(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                        int8_t* q, uint16_t* scales_f16)
{
    qg::Layout L;
    if (!packed || !q || !scales_f16) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q8G64, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    const int64_t groups = K / 64;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    const int64_t n = row_of(L, t, r, rho);
                    if (n >= N) continue;
                    const int64_t u = j * L.G + g;
                    const uint8_t* src = p + code_off(L, t, j, r, lane);
                    for (int b = 0; b < 16; ++b) q[n * K + u * 16 + b] = int8_t(int(src[b]) - 128);
                    if (g % 4 == 0)
                        memcpy(&scales_f16[n * groups + u / 4], p + meta_off_q8(L, t, j, r, rho, g / 4), 2);
                }
    return QG_OK;
}

qg_status qpack_q4g32(const uint8_t* codes, const uint16_t* scales_f16, const uint16_t* mins_f16,
                      int64_t N, int64_t K, void* out, size_t out_bytes)
{
    qg::Layout L;
    if (!codes || !scales_f16 || !mins_f16 || !out) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (out_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    uint8_t* o = static_cast<uint8_t*>(out);
    memset(o, 0, size_t(L.total_bytes));  // padding: code 0, scale 0, min 0
    const int64_t groups = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    const int64_t n = row_of(L, t, r, rho);
                    if (n >= N) continue;
                    const int64_t u = j * L.G + g;
                    q4_unit_pack(codes + n * (K / 2) + u * 16, o + code_off(L, t, j, r, lane));
                    const uint32_t meta = uint32_t(scales_f16[n * groups + u]) |
                                          (uint32_t(mins_f16[n * groups + u]) << 16);
                    memcpy(o + meta_off_q4(L, t, j, r, lane), &meta, 4);
                }
    return QG_OK;
}

qg_status qunpack_q4g32(const void* packed, size_t packed_bytes, int64_t N, int64_t K,
                        uint8_t* codes, uint16_t* scales_f16, uint16_t* mins_f16)
{
    qg::Layout L;
    if (!packed || !codes || !scales_f16 || !mins_f16) return QG_ERR_INVALID_ARG;
    if (!qg::make_layout(qg::FMT_Q4G32, N, K, &L)) return QG_ERR_INVALID_ARG;
    if (packed_bytes < size_t(L.total_bytes)) return QG_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed);
    const int64_t groups = K / 32;
    for (int64_t t = 0; t < L.tiles; ++t)
        for (int64_t j = 0; j < L.J; ++j)
            for (int r = 0; r < L.R; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int g = lane % L.G, rho = lane / L.G;
                    const int64_t n = row_of(L, t, r, rho);
                    if (n >= N) continue;
                    const int64_t u = j * L.G + g;
                    q4_unit_unpack(p + code_off(L, t, j, r, lane), codes + n * (K / 2) + u * 16);
                    uint32_t meta;
                    memcpy(&meta, p + meta_off_q4(L, t, j, r, lane), 4);
                    scales_f16[n * groups + u] = uint16_t(meta & 0xffff);
                    mins_f16[n * groups + u] = uint16_t(meta >> 16);
                }
    return QG_OK;
}

}  // extern "C"
