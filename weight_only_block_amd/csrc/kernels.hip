// Block-quantized decode GEMV kernels for gfx950 (CDNA4, wave64).
//
// The operation (y = W x for one to four bf16 activation rows, with W held
// as Q8G64 or Q4G32 codes) and why it is bound by the weight stream come
// from the "Decode 只有一行" and "W8 直读" (W8 direct read) sections of the
// zLLM GLM-5.3 ROCm decode post and the W4A16 reading in the commit log of
// vllm.cpp pull request #1936: the weights are consumed in their packed
// form and widened only in registers next to the multiply.  The kernel
// shape is this library's own, for MI355X:
//
//  * Every lane streams 16-byte units with one global load each; a
//    wave-wide load is one contiguous 1 KiB block of the packed buffer
//    (layout.h), read exactly once per call.
//  * The activation rows are staged once per work-group in LDS together
//    with fp32 sums of x over each 16/32-element unit.
//  * Codes become bf16 pairs in registers without a float conversion per
//    nibble: a 4-bit code c OR-ed into the bf16 pattern 0x4300 is the
//    number 128 + c, and an int8 code q is stored biased as u = q + 128 and
//    widened with the byte-to-float conversion.  A v_dot2 bf16 chain then
//    forms D = sum (c + 128) x over the unit, and the bias comes back out
//    exactly as D - 128 * X with X = sum x over the unit, accumulated with
//    the same v_dot2 chain so that an all-zero unit gives exactly zero.
//  * Per unit:  Q8  acc += s * (D - 128 X)
//               Q4  acc += s * (D - 128 X) + min * X
//  * G lanes share a row; their partial sums meet in a butterfly across
//    the lane group at the end of the tile.  No atomics: the result is the
//    same bits on every run.
// MFMA is not used: at m <= 4 there is no matrix to feed it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace qg {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                  // waves per work-group
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0)
constexpr uint32_t kMagicBf16x2 = 0x43004300u;  // (128.0, 128.0)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float half_lo(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}

__device__ __forceinline__ float half_hi(uint32_t w)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__device__ __forceinline__ u32x4 load_stream16(const uint8_t* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Meta words a lane reads per step: Q8 R fp16 scales, Q4 R (scale|min<<16).
template <int BYTES> struct Meta;
template <> struct Meta<2> {
    uint32_t w[1];
    __device__ __forceinline__ void load(const uint8_t* p) { w[0] = *reinterpret_cast<const uint16_t*>(p); }
};
template <> struct Meta<4> {
    uint32_t w[1];
    __device__ __forceinline__ void load(const uint8_t* p) { w[0] = *reinterpret_cast<const uint32_t*>(p); }
};
template <> struct Meta<8> {
    uint32_t w[2];
    __device__ __forceinline__ void load(const uint8_t* p)
    {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    }
};
template <> struct Meta<16> {
    uint32_t w[4];
    __device__ __forceinline__ void load(const uint8_t* p)
    {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
};

// 16 biased int8 codes -> 8 bf16 pairs, in x order (codes 2t, 2t+1 -> pair t).
__device__ __forceinline__ void q8_pairs(const u32x4& c, uint32_t (&pr)[8])
{
    const uint32_t v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float f0 = (float)(v[d] & 0xffu);
        const float f1 = (float)((v[d] >> 8) & 0xffu);
        const float f2 = (float)((v[d] >> 16) & 0xffu);
        const float f3 = (float)(v[d] >> 24);
        // An integer 0..255 has at most 8 significant bits, so the top half
        // of its fp32 pattern is exactly its bf16 pattern.
        pr[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        pr[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
}

// 32 reordered 4-bit codes -> 16 bf16 pairs (128 + c), in x order.
__device__ __forceinline__ void q4_pairs(const u32x4& c, uint32_t (&pr)[16])
{
    const uint32_t v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int p = 0; p < 4; ++p) pr[4 * d + p] = ((v[d] >> (4 * p)) & 0x000F000Fu) | kMagicBf16x2;
    }
}

template <int FMT, int M, int G, int R, bool GROUPED>
__global__ __launch_bounds__(kThreads) void qgemv_tile(const KernelParams p)
{
    extern __shared__ __align__(16) uint32_t lds[];
    constexpr int UD = FMT == FMT_Q8G64 ? 8 : 16;      // x dwords per unit
    constexpr int RPS = 64 / G;                        // rows per row slot
    constexpr int TR = R * RPS;                        // rows per tile
    constexpr int META_BYTES = FMT == FMT_Q8G64 ? 2 * R : 4 * R;
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G must be a power of two <= 64");
    static_assert(FMT != FMT_Q8G64 || G >= 4, "Q8 lane groups span whole 64-code groups");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane & (G - 1);
    const int rho = lane / G;
    const int KD = p.K >> 1;                           // x dwords per row
    const int U = p.K / (FMT == FMT_Q8G64 ? 16 : 32);  // units per row
    uint32_t* xs = lds;                                // [M][KD] bf16 pairs
    float* xsum = reinterpret_cast<float*>(lds + M * KD);  // [M][U]

    const int slot = GROUPED ? int(blockIdx.y) : 0;
    const int64_t tile = int64_t(blockIdx.x) * kWaves + wave;
    const bool active = tile < p.tiles;
    float* y = p.y + int64_t(slot) * p.y_slot_stride;
    const uint8_t* w = p.w;
    if (GROUPED) {
        const int e = p.ids[slot];
        if (e < 0 || e >= p.n_experts) {
            // Out-of-range expert id: read no weights, report NaN outputs.
            // The whole work-group takes this branch, so no barrier is skipped
            // by part of it.
            if (active) {
                for (int idx = lane; idx < TR; idx += 64) {
                    const int64_t row = tile * TR + idx;
                    if (row < p.N) y[row] = __builtin_nanf("");
                }
            }
            return;
        }
        w += int64_t(e) * p.expert_stride;
    }
    const uint16_t* x = p.x + int64_t(slot) * p.x_slot_stride;

    // Per-lane stream pointers.  Step j, slot r: code at + (j*R + r) * 1024.
    const uint8_t* code_ptr = w + tile * p.J * (R * 1024) + lane * 16;
    int lane_meta;
    if (FMT == FMT_Q8G64) lane_meta = ((rho * (G / 4) + (g >> 2)) * R) * 2;
    else lane_meta = lane * R * 4;
    const uint8_t* meta_ptr = w + p.code_bytes + tile * p.J * p.meta_step_bytes + lane_meta;

    // Issue step 0's weight loads before the activation staging: they do
    // not depend on x, so their latency overlaps the LDS fill.
    u32x4 cur[R];
    Meta<META_BYTES> cur_meta;
    if (active) {
#pragma unroll
        for (int r = 0; r < R; ++r) cur[r] = load_stream16(code_ptr + r * 1024);
        cur_meta.load(meta_ptr);
    }

    // Stage x (M rows) into LDS, then the per-unit sums.
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const uint32_t* xr = reinterpret_cast<const uint32_t*>(x + int64_t(i) * p.ldx);
        for (int d = threadIdx.x; d < KD; d += kThreads) xs[i * KD + d] = xr[d];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * U; idx += kThreads) {
        const int i = idx / U, u = idx - i * U;
        const uint32_t* src = xs + i * KD + u * UD;
        float X = 0.0f;
#pragma unroll
        for (int d = 0; d < UD; ++d) X = dot2(src[d], kOnesBf16x2, X);
        xsum[idx] = X;
    }
    __syncthreads();
    if (!active) return;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) acc[r][i] = 0.0f;

    for (int64_t j = 0; j < p.J; ++j) {
        u32x4 nxt[R];
        Meta<META_BYTES> nxt_meta;
        if (j + 1 < p.J) {
            const uint8_t* cp = code_ptr + (j + 1) * (R * 1024);
#pragma unroll
            for (int r = 0; r < R; ++r) nxt[r] = load_stream16(cp + r * 1024);
            nxt_meta.load(meta_ptr + (j + 1) * p.meta_step_bytes);
        }
        const int u = int(j) * G + g;
        uint32_t xd[M][UD];
        float X[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const uint4* src = reinterpret_cast<const uint4*>(xs + i * KD + u * UD);
#pragma unroll
            for (int q = 0; q < UD / 4; ++q) {
                const uint4 v = src[q];
                xd[i][4 * q] = v.x; xd[i][4 * q + 1] = v.y;
                xd[i][4 * q + 2] = v.z; xd[i][4 * q + 3] = v.w;
            }
            X[i] = xsum[i * U + u];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (FMT == FMT_Q8G64) {
                const float s = (r & 1) ? half_hi(cur_meta.w[r >> 1]) : half_lo(cur_meta.w[r >> 1]);
                uint32_t pr[8];
                q8_pairs(cur[r], pr);
#pragma unroll
                for (int i = 0; i < M; ++i) {
                    float D = 0.0f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) D = dot2(pr[t], xd[i][t], D);
                    const float c = fmaf(-128.0f, X[i], D);
                    acc[r][i] = fmaf(s, c, acc[r][i]);
                }
            } else {
                const float s = half_lo(cur_meta.w[r]);
                const float mn = half_hi(cur_meta.w[r]);
                uint32_t pr[16];
                q4_pairs(cur[r], pr);
#pragma unroll
                for (int i = 0; i < M; ++i) {
                    float D = 0.0f;
#pragma unroll
                    for (int t = 0; t < 16; ++t) D = dot2(pr[t], xd[i][t], D);
                    const float c = fmaf(-128.0f, X[i], D);
                    acc[r][i] = fmaf(s, c, acc[r][i]);
                    acc[r][i] = fmaf(mn, X[i], acc[r][i]);
                }
            }
        }
        if (j + 1 < p.J) {
#pragma unroll
            for (int r = 0; r < R; ++r) cur[r] = nxt[r];
            cur_meta = nxt_meta;
        }
    }

    // Butterfly over the G lanes of each row group.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) {
            float v = acc[r][i];
#pragma unroll
            for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[r][i] = v;
        }

    // Every lane of a group now holds all R*M sums; spread the stores.
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) {
            if ((r * M + i) % G == g) {
                const int64_t row = tile * TR + r * RPS + rho;
                if (row < p.N) y[int64_t(i) * p.ldy + row] = acc[r][i];
            }
        }
}

template <int FMT, int M, int G, bool GROUPED>
hipError_t launch_variant(const KernelParams& kp, dim3 grid, size_t lds_bytes, hipStream_t stream)
{
    auto kern = qgemv_tile<FMT, M, G, kRowSlots, GROUPED>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        int(kMaxLdsBytes));
    (void)attr;
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds_bytes, stream, kp);
    return hipGetLastError();
}

template <int FMT, int M, bool GROUPED>
hipError_t launch_g(int G, const KernelParams& kp, dim3 grid, size_t lds, hipStream_t s)
{
    switch (G) {
    case 64: return launch_variant<FMT, M, 64, GROUPED>(kp, grid, lds, s);
    case 32: return launch_variant<FMT, M, 32, GROUPED>(kp, grid, lds, s);
    case 16: return launch_variant<FMT, M, 16, GROUPED>(kp, grid, lds, s);
    case 8: return launch_variant<FMT, M, 8, GROUPED>(kp, grid, lds, s);
    case 4: return launch_variant<FMT, M, 4, GROUPED>(kp, grid, lds, s);
    default: break;
    }
    if constexpr (FMT == FMT_Q4G32) {
        switch (G) {
        case 2: return launch_variant<FMT, M, 2, GROUPED>(kp, grid, lds, s);
        case 1: return launch_variant<FMT, M, 1, GROUPED>(kp, grid, lds, s);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t lds_bytes_for(const Layout& L, int m)
{
    return size_t(m) * size_t(L.K / 2 + L.U) * 4;
}

hipError_t launch(const LaunchArgs& a)
{
    const Layout& L = a.layout;
    KernelParams kp;
    kp.w = static_cast<const uint8_t*>(a.w);
    kp.expert_stride = a.expert_stride;
    kp.ids = a.ids;
    kp.n_experts = a.n_experts;
    kp.x = a.x;
    kp.ldx = a.ldx;
    kp.x_slot_stride = a.x_slot_stride;
    kp.y = a.y;
    kp.ldy = a.ldy;
    kp.y_slot_stride = a.y_slot_stride;
    kp.N = int32_t(L.N);
    kp.K = int32_t(L.K);
    kp.J = L.J;
    kp.tiles = L.tiles;
    kp.code_bytes = L.code_bytes;
    kp.meta_step_bytes = L.meta_step_bytes;
    const dim3 grid(unsigned((L.tiles + kWaves - 1) / kWaves), unsigned(a.grouped ? a.n_slots : 1));
    const size_t lds = lds_bytes_for(L, a.m);
    const hipStream_t s = a.stream;
    if (a.grouped) {
        if (L.fmt != FMT_Q4G32 || a.m != 1) return hipErrorInvalidValue;
        return launch_g<FMT_Q4G32, 1, true>(L.G, kp, grid, lds, s);
    }
    if (L.fmt == FMT_Q8G64) {
        switch (a.m) {
        case 1: return launch_g<FMT_Q8G64, 1, false>(L.G, kp, grid, lds, s);
        case 2: return launch_g<FMT_Q8G64, 2, false>(L.G, kp, grid, lds, s);
        case 3: return launch_g<FMT_Q8G64, 3, false>(L.G, kp, grid, lds, s);
        case 4: return launch_g<FMT_Q8G64, 4, false>(L.G, kp, grid, lds, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.m) {
    case 1: return launch_g<FMT_Q4G32, 1, false>(L.G, kp, grid, lds, s);
    case 2: return launch_g<FMT_Q4G32, 2, false>(L.G, kp, grid, lds, s);
    case 3: return launch_g<FMT_Q4G32, 3, false>(L.G, kp, grid, lds, s);
    case 4: return launch_g<FMT_Q4G32, 4, false>(L.G, kp, grid, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qg
