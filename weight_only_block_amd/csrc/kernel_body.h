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
//  * The activation rows are staged once per work-group in LDS, for Q4G32
//    together with two fp32 sums per 32-wide group: X = sum x and
//    XA = sum |x|.  For one row and tiles of 2, 3 or 5 steps, each lane
//    may instead hold just its own units of x (and their sums) in
//    registers, with a ring of exactly one tile (XRegs).
//  * Every output must be within 2e-3 * sum |w x| of the exact sum, for any
//    inputs (rows of zero weights must give zero, a row whose only nonzero
//    weight meets a 1e-5 activation must give that one product).
//      Q8   the signed code q is widened straight from its byte (one
//           sign-extending byte-to-float conversion; every int8 is exact in
//           bf16), and v_dot2 bf16 chains form D = sum q x over the 16-code
//           unit:  acc += s * D.  No bias enters D, so the rounding error is
//           a few fp32 ulps of sum |w x| by the usual summation bound.
//      Q4   the fast path turns each nibble pair into the bf16 pair
//           (128 + c0, 128 + c1) with one and-or (0x4300 | c is 128 + c), so
//           v_dot2 chains give D = sum (128 + c) x and, per group,
//             y_g = s (D - 128 X) + min X.
//           The bias makes the rounding error scale with 128 s XA rather
//           than with sum |w x|, so every tile carries a certificate: per
//           row, A = sum |y_g| (a lower bound of sum |w x| up to the error)
//           and E = sum (|s| + |min| / 256) XA, from which a proven error
//           bound kappa E follows (see kQ4Kappa).  When kappa E <= T A for
//           every row of the tile (T is the bar less the accumulation
//           error), the fast sums meet the bar; otherwise the wave streams
//           the tile again and recomputes it exactly: each group re-centred
//           on the integer z nearest its zero point (clamped to 0..15), the
//           differences c - z widened exactly, and
//             y_g = s * sum (c - z) x + (min + s z) X,
//           where |s (c - z)| <= 2 |w| and |min + s z| <= |w| for every
//           weight of the group, so neither term can cancel.  Ordinary data
//           never needs the second pass; zero or near-cancelling groups do.
//  * G lanes share a row; their partial sums meet in a butterfly across
//    the lane group at the end of the tile.  No atomics: the result is the
//    same bits on every run.
// MFMA is not used: at m <= 4 there is no matrix to feed it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "argmax_key.h"
#include "launch.h"

namespace qg {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0)

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
// Non-temporal like the codes: each meta word is read once per call (about
// 1% faster than plain loads on the LM head and the routed experts).
template <int BYTES> struct Meta;
template <> struct Meta<2> {
    uint32_t w[1];
    __device__ __forceinline__ void load(const uint8_t* p) { w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)); }
};
template <> struct Meta<4> {
    uint32_t w[1];
    __device__ __forceinline__ void load(const uint8_t* p) { w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
};
template <> struct Meta<8> {
    uint32_t w[2];
    __device__ __forceinline__ void load(const uint8_t* p)
    {
        const uint64_t v = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
        w[0] = uint32_t(v); w[1] = uint32_t(v >> 32);
    }
};
template <> struct Meta<16> {
    uint32_t w[4];
    __device__ __forceinline__ void load(const uint8_t* p)
    {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
};

// 16 signed int8 codes -> 8 bf16 pairs, in x order (codes 2t, 2t+1 -> pair
// t).  (float)(int8_t) of a byte is one sign-extending byte-to-float
// conversion on gfx950 (v_cvt_f32_i32 with a sign-extended byte select).
__device__ __forceinline__ void q8_pairs(const u32x4& c, uint32_t (&pr)[8])
{
    const uint32_t v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float f0 = (float)(int8_t)(v[d] & 0xffu);
        const float f1 = (float)(int8_t)((v[d] >> 8) & 0xffu);
        const float f2 = (float)(int8_t)((v[d] >> 16) & 0xffu);
        const float f3 = (float)(int8_t)(v[d] >> 24);
        // An integer in [-128, 127] has at most 8 significant bits, so the
        // top half of its fp32 pattern is exactly its bf16 pattern.
        pr[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        pr[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
}

// The two constants of the 4-bit fast decode, held in registers for the
// whole kernel: the nibble-pair mask in a scalar register and the bf16 magic
// in a vector register.  gfx9 VOP3 encodings take no literal constants, so
// with both written as literals the compiler splits every (v & mask) | magic
// into a v_and_b32 and a v_or_b32 (two VOP2 ops with literals); with the
// mask in an SGPR and the magic in a VGPR it is one v_and_or_b32 (one SGPR
// operand stays within the single constant-bus read).  Both values come out
// of asm so the compiler can neither fold them back into literals nor
// rematerialise them before each use.
struct Q4Consts {
    uint32_t mask;    // 0x000F000F, SGPR
    uint32_t magic;   // 0x43004300 = bf16 (128, 128), VGPR
    __device__ __forceinline__ static Q4Consts make()
    {
        Q4Consts k;
        asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(k.mask));
        asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(k.magic));
        return k;
    }
};

__device__ __forceinline__ uint32_t and_or(uint32_t v, const Q4Consts& k)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(k.mask), "v"(k.magic));
    return r;
}

// Fast decode: 32 reordered 4-bit codes (layout.h: dword d holds k = 8d + 2p
// in bits 4p..4p+3 and k = 8d + 2p + 1 in bits 16+4p..19+4p) -> 16 bf16
// pairs (128 + c), in x order: pair p of a dword is
// ((v >> 4p) & 0x000F000F) | 0x43004300, seven VALU ops per dword.
__device__ __forceinline__ void q4_pairs_biased(const u32x4& c, const Q4Consts& k, uint32_t (&pr)[16])
{
    const uint32_t v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int p = 0; p < 4; ++p) pr[4 * d + p] = and_or(v[d] >> (4 * p), k);
    }
}

// Zero point of a Q4 group from its meta word (scale in the low half, min
// in the high half, fp16): z = clamp(rint(-min / scale), 0, 15) (0 when
// that is not a number, e.g. scale = min = 0) and m' = min + scale z in one
// rounding.  An approximate reciprocal is enough: the re-centring argument
// only needs |z + min / scale| <= 1/2 up to a few ulps.
struct Q4Group {
    float s, mp;
    int z;
};

__device__ __forceinline__ Q4Group q4_group(uint32_t meta)
{
    Q4Group g;
    g.s = half_lo(meta);
    const float mn = half_hi(meta);
    const float t = -mn * __builtin_amdgcn_rcpf(g.s);
    // Comparisons with NaN are false, so a NaN ratio gives z = 0.
    const float z = t >= 0.5f ? (t < 15.0f ? rintf(t) : 15.0f) : 0.0f;
    g.mp = fmaf(g.s, z, mn);
    g.z = int(z);
    return g;
}

// Exact decode (the certificate's fallback): the same reordered codes ->
// 16 bf16 pairs (c - z), in x order.  Integers -15..15 are exact in bf16.
__device__ __forceinline__ void q4_pairs_centred(const u32x4& c, int z, uint32_t (&pr)[16])
{
    const uint32_t v[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float lo = float(int((v[d] >> (4 * p)) & 0xfu) - z);
            const float hi = float(int((v[d] >> (16 + 4 * p)) & 0xfu) - z);
            pr[4 * d + p] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
        }
    }
}

// Proven error bound of the Q4 fast path, per group, in units of
// (|s| + |min| / 256) * XA.  It models each v_dot2 step as erring by at most
// 3 * 2^-24 of |acc| + |p0| + |p1| (the largest error measured on gfx950
// over 2^20 random operands was 1.98 * 2^-24 of that sum), and every other
// fp32 operation as correctly rounded.  D = sum (128 + c) x is two chains
// of eight v_dot2 steps plus one add: at most 25 * 2^-24 * 143 XA.  X is
// formed the same way: 25 * 2^-24 XA, times 128 in D - 128 X.  The fma
// D - 128 X adds 2^-24 * 16 XA.  So |c_hat - sum c x| <= 6790 * 2^-24 XA, and
// y_g = s c + min X errs by at most 6790 * 2^-24 |s| XA + 26 * 2^-24 |min| XA
// + 2^-24 |y_g|; 26 / 6790 < 1/256 and the last term is counted with the
// accumulation error on the host side of the threshold.  The constant below
// is 6810 * 2^-24, which also covers the fp32 rounding of XA and of the
// certificate's own terms.
constexpr float kQ4Kappa = 6810.0f / 16777216.0f;
constexpr float kQ4MinWeight = 1.0f / 256.0f;

// q = n / d for 0 <= n < 2^20 and d >= 1, from a float reciprocal of d
// (inv_d = 1.0f / d, from the host) and one correction step: the product is
// within one of the quotient, and a runtime integer division would be a long
// emulated sequence.
__device__ __forceinline__ int div_small(int n, int d, float inv_d)
{
    int q = int(float(n) * inv_d);
    if (q * d > n) --q;
    else if ((q + 1) * d <= n) ++q;
    return q;
}

// x rows -> LDS as bf16 pairs; for Q4G32 also, per unit (group) u of row
// i, X = sum x at xsum[2 (i U + u)] and kappa * sum |x| (kQ4Kappa) at
// xsum[2 (i U + u) + 1].
// X is formed by two v_dot2 chains over ones (eight pairs each) and an add,
// exactly as the hot loop forms D, so that an all-zero group gives
// D - 128 X = 0 exactly.  The 8-bit formats need no sums.  Thread t handles
// units t, t + 256, ... of the flattened [M][U] array.  Its first unit is
// fetched before anything else the kernel loads (XStage::fetch), so that
// waiting for it does not also wait for the weight stream: vector memory
// loads complete in issue order.
template <int FMT, int M, int THREADS>
struct XStage {
    static constexpr int UD = FMT == FMT_Q4G32 ? 16 : 8;   // dwords per unit
    static constexpr bool kSums = FMT == FMT_Q4G32;
    uint32_t v[UD];
    int first;                                             // flattened unit index

    __device__ __forceinline__ void load_unit(const KernelParams& p, const uint16_t* x, int idx, int U)
    {
        // 4-byte loads: x rows only need 4-byte alignment, and x is read
        // once per work-group (from L2 after the first work-group).  With one
        // row, idx is the unit.
        const int i = M == 1 ? 0 : div_small(idx, U, p.inv_U), u = idx - i * U;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(x + int64_t(i) * p.ldx + u * (2 * UD));
#pragma unroll
        for (int d = 0; d < UD; ++d) v[d] = src[d];
    }

    __device__ __forceinline__ void store_unit(uint32_t* xs, float* xsum, int idx, int KD, int U, float inv_U)
    {
        const int i = M == 1 ? 0 : div_small(idx, U, inv_U), u = idx - i * U;
        u32x4* dst = reinterpret_cast<u32x4*>(xs + i * KD + u * UD);
#pragma unroll
        for (int q = 0; q < UD / 4; ++q) {
            u32x4 t;
            t.x = v[4 * q]; t.y = v[4 * q + 1]; t.z = v[4 * q + 2]; t.w = v[4 * q + 3];
            dst[q] = t;
        }
        if constexpr (kSums) {
            float X0 = 0.0f, X1 = 0.0f, A0 = 0.0f, A1 = 0.0f;
#pragma unroll
            for (int d = 0; d < UD / 2; ++d) {
                X0 = dot2(v[d], kOnesBf16x2, X0);
                X1 = dot2(v[d + UD / 2], kOnesBf16x2, X1);
                A0 = dot2(v[d] & 0x7fff7fffu, kOnesBf16x2, A0);
                A1 = dot2(v[d + UD / 2] & 0x7fff7fffu, kOnesBf16x2, A1);
            }
            float2 xa;
            xa.x = X0 + X1;
            xa.y = kQ4Kappa * (A0 + A1);   // kappa * sum |x|, for the certificate
            reinterpret_cast<float2*>(xsum)[idx] = xa;
        }
    }

    __device__ __forceinline__ void fetch(const KernelParams& p, const uint16_t* x, int U)
    {
        // Every lane loads (lanes past the end re-read the last unit), so the
        // number of loads in flight is the same on every path and the wait
        // for x can skip the weight loads issued after it.
        first = threadIdx.x;
        load_unit(p, x, first < M * U ? first : M * U - 1, U);
    }

    // Stores the unit fetched first.
    __device__ __forceinline__ void finish_first(uint32_t* xs, float* xsum, int KD, int U, float inv_U)
    {
        if (first < M * U) store_unit(xs, xsum, first, KD, U, inv_U);
    }

    // Loads and stores the units past the first (only when M*U > threads).
    __device__ __forceinline__ void finish_rest(const KernelParams& p, const uint16_t* x, uint32_t* xs,
                                                float* xsum, int KD, int U)
    {
        for (int idx = first + THREADS; idx < M * U; idx += THREADS) {
            load_unit(p, x, idx, U);
            store_unit(xs, xsum, idx, KD, U, p.inv_U);
        }
    }
};

// x held in registers instead of LDS (launches whose rows have few units
// per lane: J = U / G steps per tile).  Lane g of a row group uses only the
// units j G + g, j < J, of each activation row, in every tile it streams, so
// it loads those J units once, straight from memory (L2 after the first
// wave), and no work-group staging, barrier or LDS read is needed.  The
// Q4G32 sums X and kappa * sum |x| are formed exactly as XStage forms them.
template <int FMT, int M, int J>
struct XRegs {
    static constexpr int UD = FMT == FMT_Q4G32 ? 16 : 8;   // dwords per unit
    uint32_t v[J][M][UD];
    float X[J][M], XA[J][M];                               // Q4G32 only

    __device__ __forceinline__ void load(const KernelParams& p, const uint16_t* x, int g, int G)
    {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const uint16_t* src = x + int64_t(i) * p.ldx + (j * G + g) * (2 * UD);
                if (p.x_vec16) {
                    // 16-byte loads where x, its row stride and its slot
                    // stride allow them (the same in every lane).
#pragma unroll
                    for (int q = 0; q < UD / 4; ++q) {
                        const u32x4 t = *reinterpret_cast<const u32x4*>(src + 8 * q);
                        v[j][i][4 * q] = t.x; v[j][i][4 * q + 1] = t.y;
                        v[j][i][4 * q + 2] = t.z; v[j][i][4 * q + 3] = t.w;
                    }
                } else {
                    const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src);
#pragma unroll
                    for (int d = 0; d < UD; ++d) v[j][i][d] = s4[d];
                }
            }
    }

    __device__ __forceinline__ void sums()
    {
        if constexpr (FMT == FMT_Q4G32) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int i = 0; i < M; ++i) {
                    float X0 = 0.0f, X1 = 0.0f, A0 = 0.0f, A1 = 0.0f;
#pragma unroll
                    for (int d = 0; d < UD / 2; ++d) {
                        X0 = dot2(v[j][i][d], kOnesBf16x2, X0);
                        X1 = dot2(v[j][i][d + UD / 2], kOnesBf16x2, X1);
                        A0 = dot2(v[j][i][d] & 0x7fff7fffu, kOnesBf16x2, A0);
                        A1 = dot2(v[j][i][d + UD / 2] & 0x7fff7fffu, kOnesBf16x2, A1);
                    }
                    X[j][i] = X0 + X1;
                    XA[j][i] = kQ4Kappa * (A0 + A1);
                }
        }
    }
};

// One work item = one step of one tile: R 16-byte units per lane plus the
// lane's meta word(s).  Items of a matrix are laid out back to back, so item
// i of tile t has its blocks at i * R KiB and its meta at
// code_bytes + i * meta_step + t * meta_tile (layout.h).
template <int R, int META_BYTES>
struct Item {
    u32x4 c[R];
    Meta<META_BYTES> m;
    __device__ __forceinline__ void load(const uint8_t* code_lane, const uint8_t* meta_lane,
                                         int64_t item, int64_t tile, const KernelParams& p)
    {
        const uint8_t* cp = code_lane + item * (R * 1024);
#pragma unroll
        for (int r = 0; r < R; ++r) c[r] = load_stream16(cp + r * 1024);
        m.load(meta_lane + item * p.meta_step_bytes + tile * p.meta_tile_bytes);
    }
};

// The Q4 fast path's per-row certificate (see kQ4Kappa), one sum per row:
// C = sum over the groups a lane has consumed of
//     T |y_g| - kappa (|s| + |min| / 256) XA,
// with kappa folded into the staged XA.  The row's fast sum is proven to
// meet the bar when its C >= 0.
template <int FMT, int M, int R>
struct Cert {
    static constexpr bool kOn = FMT == FMT_Q4G32;
    float C[kOn ? R : 1][kOn ? M : 1];
    __device__ __forceinline__ void clear()
    {
#pragma unroll
        for (int r = 0; r < (kOn ? R : 1); ++r)
#pragma unroll
            for (int i = 0; i < (kOn ? M : 1); ++i) C[r][i] = 0.0f;
    }
};

// One item against one unit of each activation row: xd holds the unit's x
// pairs, X and XA its Q4 sums (X = sum x, XA = kappa * sum |x|).
template <int FMT, int M, int R, int META_BYTES, int UD>
__device__ __forceinline__ void consume_x(const Item<R, META_BYTES>& it, const uint32_t (&xd)[M][UD],
                                          const float (&X)[M], const float (&XA)[M], const Q4Consts& k4,
                                          float T, float (&acc)[R][M], Cert<FMT, M, R>& cert)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if constexpr (FMT != FMT_Q4G32) {
            // Q8G64/Q8G128: fp16 scale of the unit's group; Q8PC: fp32 row scale.
            float s;
            if constexpr (FMT == FMT_Q8PC) s = __uint_as_float(it.m.w[r]);
            else s = (r & 1) ? half_hi(it.m.w[r >> 1]) : half_lo(it.m.w[r >> 1]);
            uint32_t pr[8];
            q8_pairs(it.c[r], pr);
#pragma unroll
            for (int i = 0; i < M; ++i) {
                float D = 0.0f;
#pragma unroll
                for (int t = 0; t < 8; ++t) D = dot2(pr[t], xd[i][t], D);
                acc[r][i] = fmaf(s, D, acc[r][i]);
            }
        } else {
            const float s = half_lo(it.m.w[r]);
            const float mn = half_hi(it.m.w[r]);
            const float we = fmaf(fabsf(mn), kQ4MinWeight, fabsf(s));
            uint32_t pr[16];
            q4_pairs_biased(it.c[r], k4, pr);
#pragma unroll
            for (int i = 0; i < M; ++i) {
                // Two chains of eight pairs (the certificate's bound assumes
                // this shape, and so does the X sum staged with x).
                float D0 = 0.0f, D1 = 0.0f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    D0 = dot2(pr[t], xd[i][t], D0);
                    D1 = dot2(pr[t + 8], xd[i][t + 8], D1);
                }
                const float c = fmaf(-128.0f, X[i], D0 + D1);
                const float yg = fmaf(s, c, mn * X[i]);
                acc[r][i] += yg;
                cert.C[r][i] = fmaf(T, fabsf(yg), cert.C[r][i]);
                cert.C[r][i] = fmaf(-we, XA[i], cert.C[r][i]);
            }
        }
    }
}

// The same with the unit's x read from the work-group's LDS copy.
template <int FMT, int M, int R, int META_BYTES>
__device__ __forceinline__ void consume(const Item<R, META_BYTES>& it, const uint32_t* xs,
                                        const float* xsum, int KD, int U, int u, const Q4Consts& k4,
                                        float T, float (&acc)[R][M], Cert<FMT, M, R>& cert)
{
    constexpr int UD = FMT == FMT_Q4G32 ? 16 : 8;
    uint32_t xd[M][UD];
    float X[M], XA[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const u32x4* src = reinterpret_cast<const u32x4*>(xs + i * KD + u * UD);
#pragma unroll
        for (int q = 0; q < UD / 4; ++q) {
            const u32x4 v = src[q];
            xd[i][4 * q] = v.x; xd[i][4 * q + 1] = v.y;
            xd[i][4 * q + 2] = v.z; xd[i][4 * q + 3] = v.w;
        }
        if constexpr (FMT == FMT_Q4G32) {
            const float2 xa = reinterpret_cast<const float2*>(xsum)[i * U + u];
            X[i] = xa.x;
            XA[i] = xa.y;
        } else {
            X[i] = XA[i] = 0.0f;
        }
    }
    consume_x<FMT, M, R, META_BYTES, UD>(it, xd, X, XA, k4, T, acc, cert);
}

// The certificate's fallback: one item of a Q4 tile, decoded exactly (each
// group re-centred on its integer zero point z, see q4_group), against x
// pairs xd and sums X of one unit per activation row.
template <int M, int R, int META_BYTES>
__device__ __forceinline__ void consume_centred_x(const Item<R, META_BYTES>& it, const uint32_t (&xd)[M][16],
                                                  const float (&X)[M], float (&acc)[R][M])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const Q4Group q = q4_group(it.m.w[r]);
        uint32_t pr[16];
        q4_pairs_centred(it.c[r], q.z, pr);
#pragma unroll
        for (int i = 0; i < M; ++i) {
            float D = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t) D = dot2(pr[t], xd[i][t], D);
            acc[r][i] = fmaf(q.s, D, acc[r][i]);
            acc[r][i] = fmaf(q.mp, X[i], acc[r][i]);
        }
    }
}

template <int M, int R, int META_BYTES>
__device__ __forceinline__ void consume_centred(const Item<R, META_BYTES>& it, const uint32_t* xs,
                                                const float* xsum, int KD, int U, int u,
                                                float (&acc)[R][M])
{
    uint32_t xd[M][16];
    float X[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const u32x4* src = reinterpret_cast<const u32x4*>(xs + i * KD + u * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 v = src[q];
            xd[i][4 * q] = v.x; xd[i][4 * q + 1] = v.y;
            xd[i][4 * q + 2] = v.z; xd[i][4 * q + 3] = v.w;
        }
        X[i] = reinterpret_cast<const float2*>(xsum)[i * U + u].x;
    }
    consume_centred_x<M, R, META_BYTES>(it, xd, X, acc);
}

__device__ __forceinline__ float dpp_add(float v, int ctrl_sel)
{
    int t;
    const int bits = __builtin_bit_cast(int, v);
    switch (ctrl_sel) {
    case 0: t = __builtin_amdgcn_update_dpp(0, bits, 0xB1, 0xf, 0xf, false); break;   // lane ^ 1
    case 1: t = __builtin_amdgcn_update_dpp(0, bits, 0x4E, 0xf, 0xf, false); break;   // lane ^ 2
    case 2: t = __builtin_amdgcn_update_dpp(0, bits, 0x141, 0xf, 0xf, false); break;  // 7 - lane in 8
    default: t = __builtin_amdgcn_update_dpp(0, bits, 0x140, 0xf, 0xf, false); break; // 15 - lane in 16
    }
    return v + __builtin_bit_cast(float, t);
}

// Sum over the 32-lane halves (BIT 5) or the 16-lane rows (BIT 4) of two
// registers at once: lanes whose BIT is 0 get a's sum, the others b's.
template <int BIT>
__device__ __forceinline__ float swap_add(float a, float b)
{
    const int ia = __builtin_bit_cast(int, a), ib = __builtin_bit_cast(int, b);
    // The two results are copied into plain locals before use: with this
    // compiler, bit-casting s[1] straight out of a const result vector is
    // lowered as s[0] (seen in the generated IR), which loses half the sum.
    unsigned lo, hi;
    if constexpr (BIT == 5) {
        auto s = __builtin_amdgcn_permlane32_swap(ia, ib, false, false);
        lo = s[0];
        hi = s[1];
    } else {
        auto s = __builtin_amdgcn_permlane16_swap(ia, ib, false, false);
        lo = s[0];
        hi = s[1];
    }
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// All-lane sum over lane bit BIT of one register.
template <int BIT>
__device__ __forceinline__ float bit_add(float v)
{
    if constexpr (BIT >= 4) return swap_add<BIT>(v, v);
    else return dpp_add(v, BIT);
}

// End of a tile: sum each of the V = R*M accumulators over the G lanes of its
// row group (lane bits 0 .. log2 G - 1).  With G >= 32 the top lane bits are
// summed as a transpose: one swap + one add folds two accumulators at once,
// after which lanes differ in which accumulator they hold (bit 5 / bit 4 of
// the lane picks it).  The remaining bits are plain butterflies (DPP inside
// a 16-lane row, swaps across rows).  Each sum is then held by the lanes
// whose untransposed group bits are zero.
template <int M, int G, int R>
struct TileSums {
    static constexpr int V = R * M;
    static constexpr int LOGG = G >= 64 ? 6 : G >= 32 ? 5 : G >= 16 ? 4 : G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0;
    static constexpr bool T5 = LOGG == 6 && V % 2 == 0;        // transpose on lane bit 5
    static constexpr int V1 = T5 ? V / 2 : V;
    static constexpr bool T4 = LOGG >= 5 && V1 % 2 == 0;       // transpose on lane bit 4
    static constexpr int V2 = T4 ? V1 / 2 : V1;
    float v[V2];

    // Accumulator index (r * M + i) whose sum this lane holds in v[k].
    __device__ __forceinline__ static int which(int k, int lane)
    {
        const int b5 = (lane >> 5) & 1, b4 = (lane >> 4) & 1;
        if constexpr (T5 && T4) return 4 * k + 2 * b4 + b5;
        else if constexpr (T5) return 2 * k + b5;
        else if constexpr (T4) return 2 * k + b4;
        else return k;
    }

    // Lanes that hold complete sums (one per row group and accumulator).
    __device__ __forceinline__ static bool holder(int g)
    {
        int transposed_mask = 0;
        if constexpr (T5) transposed_mask |= 32;
        if constexpr (T4) transposed_mask |= 16;
        return (g & ~transposed_mask) == 0;
    }
};

template <int M, int G, int R>
__device__ __forceinline__ void reduce_tile(float (&acc)[R][M], TileSums<M, G, R>& out)
{
    using TS = TileSums<M, G, R>;
    float v0[TS::V];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) {
            v0[r * M + i] = acc[r][i];
            acc[r][i] = 0.0f;
        }
    float v1[TS::V1];
    if constexpr (TS::T5) {
#pragma unroll
        for (int k = 0; k < TS::V1; ++k) v1[k] = swap_add<5>(v0[2 * k], v0[2 * k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < TS::V1; ++k) v1[k] = TS::LOGG == 6 ? bit_add<5>(v0[k]) : v0[k];
    }
    if constexpr (TS::T4) {
#pragma unroll
        for (int k = 0; k < TS::V2; ++k) out.v[k] = swap_add<4>(v1[2 * k], v1[2 * k + 1]);
    } else {
#pragma unroll
        for (int k = 0; k < TS::V2; ++k) out.v[k] = TS::LOGG >= 5 ? bit_add<4>(v1[k]) : v1[k];
    }
#pragma unroll
    for (int k = 0; k < TS::V2; ++k) {
        if constexpr (TS::LOGG >= 4) out.v[k] = bit_add<3>(out.v[k]);
        if constexpr (TS::LOGG >= 3) out.v[k] = bit_add<2>(out.v[k]);
        if constexpr (TS::LOGG >= 2) out.v[k] = bit_add<1>(out.v[k]);
        if constexpr (TS::LOGG >= 1) out.v[k] = bit_add<0>(out.v[k]);
    }
}

// Reduces the tile and stores its fp32 sums.
template <int M, int G, int R>
__device__ __forceinline__ void finish_tile(float (&acc)[R][M], const KernelParams& p, float* y,
                                            int64_t tile, int g, int rho, int lane)
{
    constexpr int RPS = 64 / G;
    constexpr int TR = R * RPS;
    TileSums<M, G, R> ts;
    reduce_tile<M, G, R>(acc, ts);
    const bool holder = TileSums<M, G, R>::holder(g);
#pragma unroll
    for (int k = 0; k < TileSums<M, G, R>::V2; ++k) {
        const int o = TileSums<M, G, R>::which(k, lane);
        const int r = o / M, i = o - (o / M) * M;
        const int64_t row = tile * TR + r * RPS + rho;
        if (holder && row < p.N) y[int64_t(i) * p.ldy + row] = ts.v[k];
    }
}

// End of a Q4 tile: reduces the certificate sum of every row the tile holds
// and reports whether each row's fast sums are proven to meet the bar
// (C >= 0; false for NaN).  The answer is the same in every lane of the
// wave (a ballot), so the caller branches uniformly.
template <int M, int G, int R>
__device__ __forceinline__ bool q4_tile_certified(Cert<FMT_Q4G32, M, R>& cert, int g)
{
    using TS = TileSums<M, G, R>;
    TS tc;
    reduce_tile<M, G, R>(cert.C, tc);
    bool bad = false;
    if (TS::holder(g)) {
#pragma unroll
        for (int k = 0; k < TS::V2; ++k) bad = bad || !(tc.v[k] >= 0.0f);
    }
    return __builtin_amdgcn_ballot_w64(bad) == 0;
}

// The certificate's fallback: the tile's J items are streamed again, one at
// a time, and its sums recomputed exactly (consume_centred).  Items are
// addressed as in the main stream, so every load stays inside the matrix.
template <int M, int G, int R, int META_BYTES>
__device__ __forceinline__ void q4_recompute_tile(float (&acc)[R][M], const KernelParams& p,
                                                  const uint8_t* code_lane, const uint8_t* meta_lane,
                                                  int64_t tile, const uint32_t* xs, const float* xsum,
                                                  int KD, int U, int g)
{
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) acc[r][i] = 0.0f;
    for (int64_t jj = 0; jj < p.J; ++jj) {
        Item<R, META_BYTES> it;
        it.load(code_lane, meta_lane, tile * p.J + jj, tile, p);
        consume_centred<M, R, META_BYTES>(it, xs, xsum, KD, U, int(jj) * G + g, acc);
    }
}

// The same with x held in registers (J steps per tile, known at compile time).
template <int M, int R, int META_BYTES, int J>
__device__ __forceinline__ void q4_recompute_tile_xr(float (&acc)[R][M], const KernelParams& p,
                                                     const uint8_t* code_lane, const uint8_t* meta_lane,
                                                     int64_t tile, const XRegs<FMT_Q4G32, M, J>& xr)
{
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) acc[r][i] = 0.0f;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
        Item<R, META_BYTES> it;
        it.load(code_lane, meta_lane, tile * J + jj, tile, p);
        consume_centred_x<M, R, META_BYTES>(it, xr.v[jj], xr.X[jj], acc);
    }
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t to_bf16(float v)
{
    const uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) return uint16_t(0x7fc0);
    return uint16_t((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

// Gate/up pair layout (layout.h): row slot 0 of a tile holds gate rows and
// slot 1 the up rows with the same output indices.  A tile yields only 64/G
// outputs, so running silu, the bf16 rounding and the store once per tile
// would cost a whole wave's issue slots for one or two values.  Instead the
// reduced sums of up to B consecutive tiles wait in registers, tile b of the
// batch in the lanes whose low bits equal b (after reduce_tile every lane of
// a row group holds the full sum, so B is the number of lanes sharing a
// value: G, or G/2 when the gate and up sums were transposed onto lane bit 5
// or 4), and one pass over the batch writes bf16(silu(g) * u) for all of them.
template <int G, int R>
struct SwigluBatch {
    static_assert(R == 2, "gate and up occupy the two row slots");
    using TS = TileSums<1, G, R>;
    static constexpr int RPS = 64 / G;
    static constexpr int B = (TS::T5 || TS::T4) ? G / 2 : G;
    float v0 = 0.0f, v1 = 0.0f;   // this lane's batch entry (gate|up, or gate and up)
    int n = 0;                    // tiles in the batch (the same in every lane)
    int64_t first = 0;            // tile index of batch entry 0

    __device__ __forceinline__ bool full() const { return n == B; }

    __device__ __forceinline__ void add(float (&acc)[R][1], int64_t tile, int lane)
    {
        TS ts;
        reduce_tile<1, G, R>(acc, ts);
        if (n == 0) first = tile;
        if ((lane & (B - 1)) == n) {
            v0 = ts.v[0];
            if constexpr (TS::V2 == 2) v1 = ts.v[1];
        }
        ++n;
    }

    // Writes the batch (tiles first, first + tstep, ...) and empties it.
    __device__ __forceinline__ void flush(const KernelParams& p, uint16_t* act, int64_t tstep, int lane,
                                          int rho)
    {
        float gate, up;
        bool writer = true;
        if constexpr (TS::V2 == 1) {
            // One transposed bit separates the gate lanes (bit clear) from the up lanes.
            constexpr int BIT = TS::T5 ? 32 : 16;
            const float other = __shfl_xor(v0, BIT, 64);
            const bool is_up = (lane & BIT) != 0;
            gate = is_up ? other : v0;
            up = is_up ? v0 : other;
            writer = !is_up;
        } else {
            gate = v0;
            up = v1;
        }
        const int b = lane & (B - 1);
        const int64_t row = (first + int64_t(b) * tstep) * RPS + rho;
        if (writer && b < n && row < p.n_out) {
            // sigmoid(g) from e = exp(-|g|) <= 1, so exp never overflows: for a
            // very negative gate silu(g) = g e^g / (1 + e^g) stays a tiny
            // nonzero number instead of g / inf.
            const float e = expf(-fabsf(gate));
            const float sig = (gate >= 0.0f ? 1.0f : e) / (1.0f + e);
            act[row] = to_bf16(gate * sig * up);
        }
        n = 0;
    }
};

// Argmax epilogue: reduces the tile like finish_tile, stores the logits if
// the caller wants them, and folds each finished logit into the lane's
// running key for its activation row.
template <int M, int G, int R>
__device__ __forceinline__ void finish_tile_argmax(float (&acc)[R][M], const KernelParams& p, float* y,
                                                   int64_t tile, int g, int rho, int lane,
                                                   uint64_t (&best)[M])
{
    constexpr int RPS = 64 / G;
    constexpr int TR = R * RPS;
    TileSums<M, G, R> ts;
    reduce_tile<M, G, R>(acc, ts);
    const bool holder = TileSums<M, G, R>::holder(g);
#pragma unroll
    for (int k = 0; k < TileSums<M, G, R>::V2; ++k) {
        const int o = TileSums<M, G, R>::which(k, lane);
        const int r = o / M, i = o - (o / M) * M;
        const int64_t row = tile * TR + r * RPS + rho;
        if (holder && row < p.N) {
            if (y) y[int64_t(i) * p.ldy + row] = ts.v[k];
            const uint64_t key = argmax_key(ts.v[k], uint32_t(row));
#pragma unroll
            for (int ii = 0; ii < M; ++ii)
                if (ii == i) best[ii] = max_key(best[ii], key);
        }
    }
}

// End of an argmax-epilogue launch: the work-group's best key per row goes
// into the row's global key with an atomic max (order-free, so the result
// is the same whatever the timing); the last work-group to finish writes
// the indices and zeroes the keys and the counter for the next call.
template <int M>
__device__ __forceinline__ void finish_argmax(uint64_t (&best)[M], const KernelParams& p, int lane, int wave)
{
    __shared__ uint64_t wave_best[4][M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const unsigned long long o = __shfl_xor((unsigned long long)best[i], off, 64);
            best[i] = max_key(best[i], o);
        }
        if (lane == 0) wave_best[wave][i] = best[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < M; ++i) {
            uint64_t k = wave_best[0][i];
#pragma unroll
            for (int w = 1; w < 4; ++w) k = max_key(k, wave_best[w][i]);
            atomicMax(&p.keys[i], (unsigned long long)k);
        }
        // The maxima are performed before this work-group counts itself.
        // Keys are read back only through atomics, so a wait for the
        // atomics (not a fence, which writes back and invalidates the whole
        // L2) is all the ordering needed.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const unsigned int done = atomicAdd(p.counter, 1u);
        if (done == gridDim.x - 1) {
#pragma unroll
            for (int i = 0; i < M; ++i) p.idx_out[i] = key_index(atomicExch(&p.keys[i], 0ull));
            atomicExch(p.counter, 0u);
        }
    }
}

// Waves sweep the matrix together: global wave gw of a slot streams tiles
// gw, gw + W, gw + 2W, ... (W = waves per slot), so at any moment the whole
// launch reads one contiguous window of the packed buffer.  That keeps the
// HBM page locality of a plain linear read; giving each wave its own
// contiguous region instead spreads the concurrent requests over the whole
// matrix and measurably loses bandwidth.  Every wave gets the same number of
// tiles up to one.  The work-group stages x once for its waves, and a ring of
// DEPTH items in registers keeps up to DEPTH*R KiB of loads in flight per wave.
// EPI 0 stores fp32 sums; EPI 1 is the SwiGLU epilogue over gate/up pairs
// (grouped Q4G32, m = 1 only); EPI 2 is the greedy argmax epilogue (dense,
// logits store optional).
// One per-wave timeline record (qg_set_wave_trace), written by lane 0 as
// the wave ends: start, first weights in and end times (s_memrealtime, a
// constant 100 MHz clock), the hardware and XCC ids, slot, wave index in
// the slot and the launch's index.
__device__ __forceinline__ void trace_wave(const KernelParams& p, uint64_t t_start, uint64_t t_first,
                                           int slot, int64_t gw, int lane)
{
    if (!p.trace || lane != 0) return;
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int64_t per_slot = int64_t(gridDim.x) * int64_t(blockDim.x >> 6);
    unsigned long long* r = p.trace + (int64_t(slot) * per_slot + gw) * 8;
    r[0] = t_start;
    r[1] = t_first;
    r[2] = __builtin_amdgcn_s_memrealtime();
    r[3] = hw;
    r[4] = xcc;
    r[5] = uint64_t(slot);
    r[6] = uint64_t(gw);
    r[7] = uint64_t(p.trace_launch);
}

template <int FMT, int M, int G, int R, int DEPTH, int WAVES, bool GROUPED, int EPI, int XRJ, bool TRACE>
__global__ __launch_bounds__(64 * WAVES) void qgemv_stream(const KernelParams p)
{
    // XRJ > 0: x in registers (XRegs) for rows of exactly XRJ steps per tile;
    // the ring then holds whole tiles, so each slot always holds the same
    // step and indexes x at compile time.
    static_assert(XRJ == 0 || DEPTH % XRJ == 0, "with x in registers the ring holds whole tiles");
    constexpr int kWaves = WAVES;
    constexpr int kThreads = 64 * WAVES;
    extern __shared__ __align__(16) uint32_t lds[];
    // Meta bytes a lane reads per item: R fp16 scales (Q8G64, Q8G128), R
    // scale|min dwords (Q4G32) or R fp32 row scales (Q8PC).
    constexpr int META_BYTES = (FMT == FMT_Q8G64 || FMT == FMT_Q8G128) ? 2 * R : 4 * R;
    constexpr int RPS = 64 / G;
    constexpr int TR = R * RPS;
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G must be a power of two <= 64");
    static_assert(FMT != FMT_Q8G64 || G >= 4, "Q8G64 lane groups span whole 64-code groups");
    static_assert(FMT != FMT_Q8G128 || G >= 8, "Q8G128 lane groups span whole 128-code groups");

    const int lane = threadIdx.x & 63;
    // The wave index is the same in every lane; say so, so that all item
    // bookkeeping below lives in scalar registers and branches uniformly.
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int g = lane & (G - 1);
    const int rho = lane / G;
    const int KD = p.K >> 1;
    const int U = p.K / (FMT == FMT_Q4G32 ? 32 : 16);
    uint32_t* xs = lds;
    float* xsum = reinterpret_cast<float*>(lds + M * KD);   // Q4G32 only

    const int slot = GROUPED ? int(blockIdx.y) : 0;
    const int64_t W = int64_t(gridDim.x) * kWaves;
    const int64_t gw = int64_t(blockIdx.x) * kWaves + wave;
    // Tile mapping: grid-stride (tiles gw, gw + W, ...) or, with contig_k > 0,
    // a contiguous run of contig_k tiles per wave.
    int64_t t0, tstep, my_tiles;
    if (p.contig_k > 0) {
        t0 = gw * p.contig_k;
        tstep = 1;
        my_tiles = t0 < p.tiles ? (p.tiles - t0 < p.contig_k ? p.tiles - t0 : p.contig_k) : 0;
    } else {
        // Tiles gw, gw + W, ... below p.tiles: the host passes tiles = q W + r
        // for this grid, so the count needs no division here (a 64-bit
        // division is a long emulated sequence on the way to the first load).
        t0 = gw;
        tstep = W;
        my_tiles = p.tiles_q + (gw < p.tiles_r ? 1 : 0);
    }
    static_assert(EPI != 1 || (FMT == FMT_Q4G32 && M == 1 && GROUPED && R == 2),
                  "the SwiGLU epilogue is built for grouped Q4G32 gate/up pairs");
    static_assert(EPI != 2 || (!GROUPED && WAVES == 4), "the argmax epilogue is for dense launches");
    float* y = p.y + int64_t(slot) * p.y_slot_stride;
    uint16_t* act = p.act + int64_t(slot) * p.act_slot_stride;
    const uint16_t* x = p.x + int64_t(slot) * p.x_slot_stride;

    // Activations first (see XStage), then the expert id, then the weights.
    // The id is read with a scalar load; nothing branches on it before the
    // weight ring is issued, so the x loads go out while the id is in
    // flight instead of waiting behind it.
    XStage<FMT, M, kThreads> xstage;
    XRegs<FMT, M, (XRJ > 0 ? XRJ : 1)> xr;
    if constexpr (XRJ > 0) xr.load(p, x, g, G);
    else xstage.fetch(p, x, U);

    const uint8_t* w = p.w;
    bool bad_expert = false;
    if (GROUPED) {
        const int e = p.ids[slot];
        // Out-of-range expert id: the work-group streams nothing (the ring's
        // spare loads read the first item of expert 0, which is in bounds)
        // and reports NaN outputs below.  e is per work-group, so every
        // wave takes the same path.
        bad_expert = e < 0 || e >= p.n_experts;
        if (!bad_expert) w += int64_t(e) * p.expert_stride;
    }
    const int64_t n_items = bad_expert ? 0 : my_tiles * p.J;

    const uint8_t* code_lane = w + lane * 16;
    int lane_meta;
    if (FMT == FMT_Q8G64) lane_meta = ((rho * (G / 4) + (g >> 2)) * R) * 2;
    else if (FMT == FMT_Q8G128) lane_meta = ((rho * (G / 8) + (g >> 3)) * R) * 2;
    else if (FMT == FMT_Q8PC) lane_meta = rho * R * 4;
    else lane_meta = lane * R * 4;
    const uint8_t* meta_lane = w + p.code_bytes + lane_meta;

    // Timeline start: the wave has its arguments (and expert id) and is
    // about to issue its first weight loads.  Read only when tracing: the
    // clock read is a scalar memory operation, and any wait for scalar
    // loads would also wait for it.
    uint64_t tr_start = 0;
    if constexpr (TRACE) tr_start = __builtin_amdgcn_s_memrealtime();

    // Load cursor: (tile, step) of the next item to fetch.
    int64_t ld_tile = t0, ld_j = 0;
    Item<R, META_BYTES> ring[DEPTH];
#define QG_LOAD_NEXT(slot_)                                                                   \
    do {                                                                                      \
        ring[slot_].load(code_lane, meta_lane, ld_tile * p.J + ld_j, ld_tile, p);            \
        if (++ld_j == p.J) { ld_j = 0; ld_tile += tstep; }                                   \
    } while (0)

    // Fill the ring unconditionally: a wave with fewer than DEPTH items loads
    // item 0 of the matrix into the spare slots (never consumed), so the
    // loads in flight are the same on every path and each wait below covers
    // exactly the loads it needs.
#define QG_FILL_RING()                                                                        \
    do {                                                                                      \
        _Pragma("unroll") for (int d = 0; d < DEPTH; ++d) {                                   \
            if (d < n_items) {                                                                \
                QG_LOAD_NEXT(d);                                                              \
            } else {                                                                          \
                ring[d].load(code_lane, meta_lane, 0, 0, p);                                  \
            }                                                                                 \
        }                                                                                     \
    } while (0)
    if constexpr (XRJ > 0) {
        // The lane's own x units were loaded first; their sums wait for x
        // alone while the weights are in flight.  No barrier: nothing is
        // shared through LDS.
        QG_FILL_RING();
        xr.sums();
    } else {
        if (M * U <= kThreads) {
            // One x unit per thread at most: it was fetched first; finish
            // staging it while the weights are in flight.
            QG_FILL_RING();
            xstage.finish_first(xs, xsum, KD, U, p.inv_U);
        } else {
            // Long activations: stage all of x, then start the weight stream.
            xstage.finish_first(xs, xsum, KD, U, p.inv_U);
            xstage.finish_rest(p, x, xs, xsum, KD, U);
            QG_FILL_RING();
        }
        __syncthreads();
    }
#undef QG_FILL_RING
    uint64_t tr_first = 0;
    if constexpr (TRACE) {
        // Timeline: the time the first weights have arrived (the empty asm
        // reads a register of the first load, so the wait for it is placed
        // here; only traced launches take this branch).
        const uint32_t first = ring[0].c[0].x;
        asm volatile("" ::"v"(first));
        tr_first = __builtin_amdgcn_s_memrealtime();
    }
    if (GROUPED && bad_expert) {
        for (int64_t n = 0, t = t0; n < my_tiles; ++n, t += tstep) {
            if constexpr (EPI == 1) {
                for (int idx = lane; idx < RPS; idx += 64) {
                    const int64_t row = t * RPS + idx;
                    if (row < p.n_out) act[row] = uint16_t(0x7fc0);
                }
            } else {
                for (int idx = lane; idx < TR; idx += 64) {
                    const int64_t row = t * TR + idx;
                    if (row < p.N) y[row] = __builtin_nanf("");
                }
            }
        }
        if constexpr (TRACE) trace_wave(p, tr_start, tr_first, slot, gw, lane);
        return;
    }
    // (The argmax epilogue needs every wave at its closing barrier.)
    if (EPI != 2 && n_items == 0) {
        if constexpr (TRACE) trace_wave(p, tr_start, tr_first, slot, gw, lane);
        return;
    }
    uint64_t best[M];
#pragma unroll
    for (int i = 0; i < M; ++i) best[i] = 0;

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < M; ++i) acc[r][i] = 0.0f;
    Q4Consts k4 = {0u, 0u};
    if constexpr (FMT == FMT_Q4G32) k4 = Q4Consts::make();
    SwigluBatch<G, R> swb;   // EPI 1 only
    Cert<FMT, M, R> cert;    // Q4G32 only
    cert.clear();

    // Consume cursor.
    int64_t tile = t0, j = 0;
#define QG_CONSUME(slot_)                                                                     \
    do {                                                                                      \
        if constexpr (XRJ > 0)                                                                \
            consume_x<FMT, M, R, META_BYTES, XRegs<FMT, M, 1>::UD>(                           \
                ring[slot_], xr.v[(slot_) % XRJ], xr.X[(slot_) % XRJ], xr.XA[(slot_) % XRJ], k4, \
                p.cert_t, acc, cert);                                                         \
        else                                                                                  \
            consume<FMT, M, R, META_BYTES>(ring[slot_], xs, xsum, KD, U, int(j) * G + g, k4,  \
                                           p.cert_t, acc, cert);                              \
    } while (0)
#define QG_ADVANCE()                                                                          \
    do {                                                                                      \
        if (++j == p.J) {                                                                     \
            if constexpr (FMT == FMT_Q4G32) {                                                 \
                if (__builtin_expect(!q4_tile_certified<M, G, R>(cert, g), 0)) {              \
                    if constexpr (XRJ > 0)                                                    \
                        q4_recompute_tile_xr<M, R, META_BYTES, (XRJ > 0 ? XRJ : 1)>(          \
                            acc, p, code_lane, meta_lane, tile, xr);                          \
                    else                                                                      \
                        q4_recompute_tile<M, G, R, META_BYTES>(acc, p, code_lane, meta_lane,  \
                                                               tile, xs, xsum, KD, U, g);     \
                }                                                                             \
            }                                                                                 \
            if constexpr (EPI == 1) {                                                         \
                swb.add(acc, tile, lane);                                                     \
                if (swb.full()) swb.flush(p, act, tstep, lane, rho);                          \
            }                                                                                 \
            else if constexpr (EPI == 2) finish_tile_argmax<M, G, R>(acc, p, p.y, tile, g, rho, lane, best); \
            else finish_tile<M, G, R>(acc, p, y, tile, g, rho, lane);                               \
            tile += tstep;                                                                    \
            j = 0;                                                                            \
        }                                                                                     \
    } while (0)

    int64_t n = 0;
    // Steady state: every consumed slot is refilled unconditionally.
    for (; n + 2 * DEPTH <= n_items; n += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            QG_CONSUME(d);
            QG_LOAD_NEXT(d);
            QG_ADVANCE();
        }
    }
    // Tail: fewer than 2*DEPTH items remain; the first min(DEPTH, rest) are
    // already in the ring.
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (n + d < n_items) {
            QG_CONSUME(d);
            if (n + DEPTH + d < n_items) QG_LOAD_NEXT(d);
            QG_ADVANCE();
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (n + DEPTH + d < n_items) {
            QG_CONSUME(d);
            QG_ADVANCE();
        }
    }
#undef QG_LOAD_NEXT
#undef QG_CONSUME
#undef QG_ADVANCE
    if constexpr (EPI == 1) {
        if (swb.n > 0) swb.flush(p, act, tstep, lane, rho);
    }
    if constexpr (EPI == 2) finish_argmax<M>(best, p, lane, wave);
    if constexpr (TRACE) trace_wave(p, tr_start, tr_first, slot, gw, lane);
}

// Launch shape (launch.h): ring depth 2 or 4; work-groups are 4 waves.

template <int FMT, int M, int G, int DEPTH, int WAVES, bool GROUPED, int EPI, int XRJ = 0>
hipError_t launch_variant(const KernelParams& kp, int64_t waves, int slots, size_t lds_bytes,
                          hipStream_t stream)
{
    auto kern = qgemv_stream<FMT, M, G, kRowSlots, DEPTH, WAVES, GROUPED, EPI, XRJ, false>;
    // The timeline records (qg_set_wave_trace) come from a separate
    // instantiation, so the untraced kernel carries no trace code at all;
    // built for one activation row only.
    auto kern_traced = qgemv_stream<FMT, M, G, kRowSlots, DEPTH, WAVES, GROUPED, EPI, XRJ, (M == 1)>;
    // Raise the dynamic-LDS limit once per kernel (static LDS is within the
    // reserve).  A failure is not left behind as the launch's error; it only
    // matters to launches that need more than the default 64 KiB.
    static const hipError_t attr = [&] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxDynLdsBytes));
        if (e == hipSuccess && M == 1)
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern_traced),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxDynLdsBytes));
        if (e != hipSuccess) (void)hipGetLastError();
        return e;
    }();
    if (attr != hipSuccess && lds_bytes > 64 * 1024) return attr;
    const dim3 grid(unsigned((waves + WAVES - 1) / WAVES), unsigned(slots));
    // The grid-stride share of each wave: tiles = q W + r for the W waves
    // of a slot (the kernel adds 1 for waves below r).
    KernelParams k = kp;
    const int64_t W = int64_t(grid.x) * WAVES;
    k.tiles_q = kp.tiles / W;
    k.tiles_r = kp.tiles % W;
    k.trace = M == 1 ? reserve_wave_trace(W * slots, &k.trace_launch) : nullptr;
    if (k.trace)
        hipLaunchKernelGGL(kern_traced, grid, dim3(64 * WAVES), lds_bytes, stream, k);
    else
        hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), lds_bytes, stream, k);
    return hipGetLastError();
}

template <int FMT, int M, int G, bool GROUPED, int EPI>
hipError_t launch_shape(int shape, const KernelParams& kp, int64_t waves, int slots, size_t lds,
                        hipStream_t s)
{
    switch (shape) {
    case SHAPE_D2_W4: return launch_variant<FMT, M, G, 2, 4, GROUPED, EPI>(kp, waves, slots, lds, s);
    case SHAPE_D4_W4: return launch_variant<FMT, M, G, 4, 4, GROUPED, EPI>(kp, waves, slots, lds, s);
    default: break;
    }
    // x in registers: built for one activation row, lane groups of 16..64
    // lanes and 2, 3 or 5 steps per tile (the ring holds one tile).
    if constexpr (M == 1 && G >= 16) {
        switch (shape) {
        case SHAPE_XR:
            switch (kp.J) {
            case 2: return launch_variant<FMT, M, G, 2, 4, GROUPED, EPI, 2>(kp, waves, slots, 0, s);
            case 3: return launch_variant<FMT, M, G, 3, 4, GROUPED, EPI, 3>(kp, waves, slots, 0, s);
            case 5: return launch_variant<FMT, M, G, 5, 4, GROUPED, EPI, 5>(kp, waves, slots, 0, s);
            default: break;
            }
            break;
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

template <int FMT, int M, bool GROUPED, int EPI>
hipError_t launch_g(int G, int shape, const KernelParams& kp, int64_t waves, int slots, size_t lds,
                    hipStream_t s)
{
    switch (G) {
    case 64: return launch_shape<FMT, M, 64, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
    case 32: return launch_shape<FMT, M, 32, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
    case 16: return launch_shape<FMT, M, 16, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
    case 8: return launch_shape<FMT, M, 8, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
    default: break;
    }
    if constexpr (FMT != FMT_Q8G128) {
        if (G == 4) return launch_shape<FMT, M, 4, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
    }
    if constexpr (FMT == FMT_Q4G32 || FMT == FMT_Q8PC) {
        switch (G) {
        case 2: return launch_shape<FMT, M, 2, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
        case 1: return launch_shape<FMT, M, 1, GROUPED, EPI>(shape, kp, waves, slots, lds, s);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Launches the kernel of format FMT for m activation rows (one instantiation
// per format, each in its own translation unit).
template <int FMT>
hipError_t launch_format(int m, bool grouped, int G, int shape, const KernelParams& kp, int64_t waves,
                         int slots, size_t lds, hipStream_t s)
{
    if (grouped) {
        if constexpr (FMT == FMT_Q4G32) {
            if (m == 1) return launch_g<FMT, 1, true, 0>(G, shape, kp, waves, slots, lds, s);
        }
        return hipErrorInvalidValue;
    }
    switch (m) {
    case 1: return launch_g<FMT, 1, false, 0>(G, shape, kp, waves, slots, lds, s);
    case 2: return launch_g<FMT, 2, false, 0>(G, shape, kp, waves, slots, lds, s);
    case 3: return launch_g<FMT, 3, false, 0>(G, shape, kp, waves, slots, lds, s);
    case 4: return launch_g<FMT, 4, false, 0>(G, shape, kp, waves, slots, lds, s);
    default: return hipErrorInvalidValue;
    }
}

// Dense launches with the argmax epilogue (m = 1..4).  A template so that
// only the translation unit that calls it instantiates the kernels.
template <int FMT>
hipError_t launch_argmax_format(int m, int G, int shape, const KernelParams& kp, int64_t waves,
                                size_t lds, hipStream_t s)
{
    switch (m) {
    case 1: return launch_g<FMT, 1, false, 2>(G, shape, kp, waves, 1, lds, s);
    case 2: return launch_g<FMT, 2, false, 2>(G, shape, kp, waves, 1, lds, s);
    case 3: return launch_g<FMT, 3, false, 2>(G, shape, kp, waves, 1, lds, s);
    case 4: return launch_g<FMT, 4, false, 2>(G, shape, kp, waves, 1, lds, s);
    default: return hipErrorInvalidValue;
    }
}

// Grouped Q4G32 gate/up pairs with the SwiGLU epilogue (m = 1).  A template
// so that only the translation unit that calls it instantiates the kernels.
template <int FMT>
hipError_t launch_swiglu(int G, int shape, const KernelParams& kp, int64_t waves, int slots,
                         size_t lds, hipStream_t s)
{
    static_assert(FMT == FMT_Q4G32, "the SwiGLU epilogue is built for Q4G32 gate/up pairs");
    return launch_g<FMT, 1, true, 1>(G, shape, kp, waves, slots, lds, s);
}

}  // namespace qg
