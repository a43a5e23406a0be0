// Batched decode GEMV (m = 2..16 activation rows) on the gfx950 matrix
// cores, for the 8-bit formats and Q4G32 in the matrix-core layout
// (layout.h, MmaLayout).  The larger-batch decode of the Qwen3 C++
// Reference Runtime (MetaInfer-cpp) README ("B8/B16" kernels with the input
// rows reused from LDS) is the operation; with up to 16 rows sharing each
// weight the dot products become a 16 x 16 x 32 bf16 matrix product per 32
// of K (two per 64-wide step of the 8-bit formats, four per 128-wide step
// of Q4G32):
//
//  * A (16 x 32): the activation rows (row i = lane mod 16; rows past m
//    repeat row m - 1, whose outputs are never stored), read from LDS,
//    where x is staged once per work-group, or from memory with each item
//    when the rows are too long to stage.
//  * B (32 x 16): 16 weight rows, 16 signed codes per lane exactly as one
//    wave load brings them in (the layout puts row lane mod 16, k-slice
//    lane div 16 in lane order), widened to bf16 (every int8 is exact).
//  * D (16 x 16, fp32): lane l holds D[4*(l div 16) + v][l mod 16].
//
// Per scale group:  acc += s * D   (s: the row's fp16 group scale); Q8PC's
// one fp32 row scale multiplies the D of a whole tile (or of a wave's part
// of it) once, at its end.  Q4G32 re-centres each 32-group on the integer
// nearest its zero point (z = clamp(rint(-min / scale), 0, 15), m' =
// min + scale z), feeds the exact differences c - z as B, and adds the
// group's activation sum X (from a per-group table formed once per
// work-group when x is staged in LDS, else a second MFMA against an
// all-ones B):
// acc += s * D + m' * X.  No bias is left inside D, so the rounding error
// of an output stays a few fp32 ulps of sum |w x| (the same argument as the
// VALU kernels').  Each output is a complete sum when its tile ends, so
// there is no cross-lane reduction and no atomic.
//
// A 16-row tile spans all of K, so a mid-size matrix has few tiles.  With
// KSPLIT = 4 (16) the four (sixteen) waves of a work-group share each tile,
// one contiguous part of its steps each; at the tile end each wave parks
// its partial sums in LDS and, after a barrier, the work-group adds the
// parts in K order and stores (the same bits on every run and for every m).
// Sixteen waves keep four times the bytes in flight per staged copy of x,
// which matters when the staged activations leave room for one work-group
// per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace qg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

// Eight signed codes (two dwords, k order) -> eight bf16 in k order.
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi)
{
    const uint32_t v[2] = {lo, hi};
    u32x4 pr;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const float f0 = (float)(int8_t)(v[d] & 0xffu);
        const float f1 = (float)(int8_t)((v[d] >> 8) & 0xffu);
        const float f2 = (float)(int8_t)((v[d] >> 16) & 0xffu);
        const float f3 = (float)(int8_t)(v[d] >> 24);
        // The top half of the fp32 pattern of an integer -128..127 is its bf16.
        pr[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        pr[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8, pr);
}

// Eight Q4 codes (one dword, canonical order: byte b holds k = 2b in the
// low nibble and 2b + 1 in the high nibble) -> eight bf16 values c - z in k
// order.  zb is z (0..15) in every byte; guarding each byte with bit 7
// keeps the subtraction from borrowing across bytes, and clearing the guard
// leaves c - z as a two's-complement byte for the exact widening.
__device__ __forceinline__ bf16x8 widen_q4(uint32_t u, uint32_t zb)
{
    const uint32_t lo = (((u & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
    const uint32_t hi = ((((u >> 4) & 0x0F0F0F0Fu) | 0x80808080u) - zb) ^ 0x80808080u;
    u32x4 pr;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float fe = (float)(int8_t)((lo >> (8 * b)) & 0xffu);
        const float fo = (float)(int8_t)((hi >> (8 * b)) & 0xffu);
        pr[b] = __builtin_amdgcn_perm(__float_as_uint(fo), __float_as_uint(fe), 0x07060302u);
    }
    return __builtin_bit_cast(bf16x8, pr);
}

__device__ __forceinline__ float half_bits(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xffffu));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + the sum of eight bf16 values (four pairs), one v_dot2 per pair.
// The pairs are copied into plain integers before the bit casts: with
// this compiler, bit-casting the elements of a vector straight from its
// reference was lowered as four casts of element 0.
__device__ __forceinline__ float sum8(u32x4 v, float acc)
{
    uint32_t e[4];
    e[0] = v.x;
    e[1] = v.y;
    e[2] = v.z;
    e[3] = v.w;
    const bf16x2 one = __builtin_bit_cast(bf16x2, kOnesBf16x2);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e[q]), one, acc, false);
    return acc;
}

// LDS position (16-byte chunk) of chunk c of activation row i: chunks are
// XOR-swizzled by the row inside each 64-wide step so that the 16 rows an
// MFMA reads at one k fall into different banks.
__device__ __forceinline__ int xs_chunk(int i, int c, int chunks_per_row)
{
    return i * chunks_per_row + (c ^ (i & 7));
}

struct MmaItem {
    u32x4 c;        // 16 signed 8-bit codes, or 32 Q4 codes (one dword per 32-group)
    uint32_t s;     // fp16 scale (low half) or fp32 row scale bits (8-bit formats)
    u32x4 m4;       // Q4G32: scale | min << 16 of the row's four groups
    u32x4 a0, a1;   // the step's A fragments, when x is read from memory (XG)
    u32x4 a2, a3;   // (Q4G32: one per 32-group)
};

// Threads per work-group: four waves, or sixteen for the 16-way K split.
template <int KSPLIT>
constexpr int mma_threads()
{
    return KSPLIT == 16 ? 1024 : 256;
}

// XG: the A fragments come from memory with each item (x is read through
// the L2, once per tile) instead of from a copy of x staged in LDS; for
// m * K too large to stage (next to a K split's partial sums).  Built for
// whole tiles per wave and for the four-wave split: with sixteen waves the
// longer ring does not fit in registers.
template <int FMT, int DEPTH, int KSPLIT, bool XG>
__global__ __launch_bounds__(mma_threads<KSPLIT>()) void qgemv_mma(const MmaParams p)
{
    constexpr int kThreads = mma_threads<KSPLIT>();
    static_assert(KSPLIT == 1 || KSPLIT == kThreads / 64, "a K split spans the work-group's waves");
    extern __shared__ __align__(16) u32x4 xs[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int rho = lane & 15;      // weight row in the tile; activation row of A
    const int qs = lane >> 4;       // k-slice of the step
    const int m = p.m;
    const int64_t J = p.J;
    const int cpr = int(p.K / 8);   // 16-byte chunks per activation row
    // Steps per scale group: 1 (Q8G64), 2 (Q8G128); Q8PC scales once per
    // tile.  A Q4G32 step (128 K) holds four whole groups, so K splits fall
    // between steps there too.
    constexpr int SPG = FMT == FMT_Q8G128 ? 2 : 1;
    constexpr bool Q4 = FMT == FMT_Q4G32;
    static_assert(!(XG && KSPLIT == 16), "x from memory is built for whole tiles or four waves");

    // Tile mapping.  KSPLIT = 1: wave gw streams tiles gw, gw + W, ...  and
    // all their steps.  KSPLIT > 1: work-group b takes tiles b, b + B, ...
    // and its wave w the steps of scale groups [G w / KSPLIT,
    // G (w + 1) / KSPLIT) of each (G = groups per row).
    int64_t W, gw, j_lo, j_hi;
    if constexpr (KSPLIT == 1) {
        W = int64_t(gridDim.x) * (kThreads / 64);
        gw = int64_t(blockIdx.x) * (kThreads / 64) + wave;
        j_lo = 0;
        j_hi = J;
    } else {
        // Quarters in whole scale groups, so no group is cut between waves.
        const int64_t G = J / SPG;
        W = gridDim.x;
        gw = blockIdx.x;
        j_lo = G * wave / KSPLIT * SPG;
        j_hi = G * (wave + 1) / KSPLIT * SPG;
    }
    // tiles = q W + r (from the host): no division on the way to the first load.
    const int64_t my_tiles = p.tiles_q + (gw < p.tiles_r ? 1 : 0);
    const int64_t n_items = my_tiles * (j_hi - j_lo);

    const uint8_t* code_lane = p.w + lane * 16;
    const uint8_t* meta = p.w + p.code_bytes;
    // 16-byte loads of x when x and its row stride allow them (the same in
    // every lane), else 4-byte loads.
    const bool x_wide = ((reinterpret_cast<uintptr_t>(p.x) | uintptr_t(p.ldx * 2)) & 15u) == 0;
    auto load_x16 = [&](const uint16_t* src) {
        u32x4 v;
        if (x_wide) {
            v = *reinterpret_cast<const u32x4*>(src);
        } else {
            const uint32_t* s4 = reinterpret_cast<const uint32_t*>(src);
            v.x = s4[0]; v.y = s4[1]; v.z = s4[2]; v.w = s4[3];
        }
        return v;
    };
    // A rows past m repeat row m - 1: each output row of an MFMA depends on
    // its own A row only, and rows past m are never stored, so nothing needs
    // zeroing and no load or LDS read sits behind a per-lane branch.
    const int xrow = rho < m ? rho : m - 1;
    // Reads of the staged x: the swizzle moves chunk c of row xrow within
    // its group of 8, and a step's chunks (8 j + t, t < 8, for the 8-bit
    // formats; 16 j + u, u < 16, for Q4G32) keep their multiple of 8, so
    // each lane's places within a step are constants and a step adds j.
    const u32x4* xs_row = xs + xrow * cpr;
    const int o0 = (2 * qs) ^ (xrow & 7), o1 = (2 * qs + 1) ^ (xrow & 7);
    int oq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) oq[g] = (4 * g + qs) ^ (xrow & 7);
    // Load cursor: the step j of the next item to load and the byte offsets
    // of its code block and of its tile's meta, advanced by additions (the
    // jump to the wave's next tile is the same every time).
    struct Cursor {
        int64_t j, code, meta;
    };
    const int64_t jump_code = (W * J + j_lo - j_hi) * 1024;
    const int64_t jump_meta = W * p.meta_tile_bytes;
    auto advance = [&](Cursor& cu) {
        cu.code += 1024;
        if (++cu.j == j_hi) {
            cu.j = j_lo;
            cu.code += jump_code;
            cu.meta += jump_meta;
        }
    };
    auto load = [&](MmaItem& it, const Cursor& cu) {
        const int64_t j = cu.j;
        it.c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(code_lane + cu.code));
        const uint8_t* mt = meta + cu.meta;
        if constexpr (Q4) it.m4 = *reinterpret_cast<const u32x4*>(mt + (j * 16 + rho) * 16);
        else if (FMT == FMT_Q8PC) it.s = *reinterpret_cast<const uint32_t*>(mt + rho * 4);
        // Group scales are read once per call: non-temporal, like the codes
        // (1% on the LM head at m = 8).  A Q8PC row scale is re-read at every
        // step of its tile and stays a plain load (3% slower otherwise).
        else it.s = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(mt + ((j / SPG) * 16 + rho) * 2));
        // x from memory: row xrow (in bounds for every lane), loaded with no
        // per-lane branch (a divergent branch around the loads had made the
        // compiler keep the ring in scratch memory and wait for every load).
        if constexpr (XG && Q4) {
            // Row xrow of x, k = 128 j + 32 g + 8 qs .. + 7 for the four groups g.
            const uint16_t* src = p.x + int64_t(xrow) * p.ldx + j * 128 + qs * 8;
            it.a0 = load_x16(src);
            it.a1 = load_x16(src + 32);
            it.a2 = load_x16(src + 64);
            it.a3 = load_x16(src + 96);
        } else if constexpr (XG) {
            // Row xrow of x, k = 64 j + 16 qs .. + 15.
            const uint16_t* src = p.x + int64_t(xrow) * p.ldx + j * 64 + qs * 16;
            it.a0 = load_x16(src);
            it.a1 = load_x16(src + 8);
        }
    };

    // Activations first, then weights: vector-memory loads complete in
    // issue order, so storing the staged x waits for x alone while the
    // weight ring is already in flight.  A thread loads up to kXBatch
    // 16-byte chunks of x before it stores any (one memory latency per
    // batch); past the first batch (long rows, four-wave groups) the
    // batches also wait for the ring.  Chunks are XOR-swizzled in LDS.
    constexpr int kXBatch = 8;
    const int x_total = XG ? 0 : m * cpr;
    // Row of a flattened chunk index (< m * cpr, far below 2^20): a float
    // reciprocal and one correction instead of an emulated integer division.
    auto row_of_chunk = [&](int idx) {
        int q = int(float(idx) * p.inv_cpr);
        if (q * cpr > idx) --q;
        else if ((q + 1) * cpr <= idx) ++q;
        return q;
    };
    u32x4 xv[kXBatch];
    auto x_load = [&](int base) {
#pragma unroll
        for (int b = 0; b < kXBatch; ++b) {
            const int idx = base + b * kThreads + int(threadIdx.x);
            if (idx < x_total) {
                const int i = row_of_chunk(idx), c = idx - i * cpr;
                xv[b] = load_x16(p.x + int64_t(i) * p.ldx + c * 8);
            }
        }
    };
    auto x_store = [&](int base) {
#pragma unroll
        for (int b = 0; b < kXBatch; ++b) {
            const int idx = base + b * kThreads + int(threadIdx.x);
            if (idx < x_total) {
                const int i = row_of_chunk(idx), c = idx - i * cpr;
                xs[xs_chunk(i, c, cpr)] = xv[b];
            }
        }
    };
    x_load(0);

    // Spare ring slots load item 0 of the matrix (never consumed) so every
    // path issues the same loads.
    Cursor ld = {j_lo, (gw * J + j_lo) * 1024, gw * p.meta_tile_bytes};
    const Cursor spare = {0, 0, 0};
    MmaItem ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (d < n_items) {
            load(ring[d], ld);
            advance(ld);
        } else {
            load(ring[d], spare);
        }
    }

    x_store(0);
    for (int base = kXBatch * kThreads; base < x_total; base += kXBatch * kThreads) {
        x_load(base);
        x_store(base);
    }
    __syncthreads();
    // Q4G32 with x staged: the sums X of each activation row over each
    // 32-group, formed once per work-group from the staged copy (two chains
    // of eight v_dot2 against ones, then an add) into a [group][16 rows]
    // table after x, and read with one LDS load per group.  Rows past m are
    // not formed: their outputs are never stored.
    constexpr bool kXTable = Q4 && !XG;
    float* xtab = reinterpret_cast<float*>(xs + x_total);
    if constexpr (kXTable) {
        const int ngroups = cpr / 4;
        const float inv_ng = 4.0f * p.inv_cpr;
        for (int idx = threadIdx.x; idx < m * ngroups; idx += kThreads) {
            int i = int(float(idx) * inv_ng);
            if (i * ngroups > idx) --i;
            else if ((i + 1) * ngroups <= idx) ++i;
            const int gi = idx - i * ngroups;
            float X0 = 0.f, X1 = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                X0 = sum8(xs[xs_chunk(i, 4 * gi + c, cpr)], X0);
                X1 = sum8(xs[xs_chunk(i, 4 * gi + 2 + c, cpr)], X1);
            }
            xtab[gi * 16 + i] = X0 + X1;
        }
        __syncthreads();
    }
    // (With the K split every wave takes part in each tile's closing barrier.)
    if (KSPLIT == 1 && n_items == 0) return;
    // K split: parked partial sums, two buffers of [wave][lane][4] floats
    // after the staged activations and the sum table (one barrier per tile).
    f32x4* part = reinterpret_cast<f32x4*>(xs + x_total + (kXTable ? cpr : 0));
    int buf = 0;

    const u32x4 ones4 = {kOnesBf16x2, kOnesBf16x2, kOnesBf16x2, kOnesBf16x2};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f32x4 D = acc;
    // Group scaling deferred by one step (group formats): the last finished
    // group's D and scale, zero when none is pending.
    f32x4 D_done = acc;
    float s_done = 0.f;
    int64_t tile = gw, j = j_lo;

    auto consume = [&](const MmaItem& it) {
        if constexpr (Q4 && !XG) {
            // Per 32-group: D = sum x (c - z) (one MFMA) and X = sum x from
            // the table, then acc += s D + m' X.  The four groups' MFMAs
            // are issued first, into separate results, so that no group
            // waits for the one before it; the adds keep the group order.
            f32x4 Dq[4];
            float sq[4], mq[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, xs_row[int(j) * 16 + oq[g]]);
                const float s = half_bits(it.m4[g]);
                const float mn = half_bits(it.m4[g] >> 16);
                const float t = -mn * __builtin_amdgcn_rcpf(s);
                // z = clamp(rint(-min / scale), 0, 15), branch-free; a NaN
                // ratio gives 0 (fmaxf returns the number).
                const float z = fminf(fmaxf(rintf(t), 0.0f), 15.0f);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                Dq[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a, widen_q4(it.c[g], __builtin_amdgcn_perm(0u, uint32_t(z), 0u)), zero, 0, 0, 0);
                sq[g] = s;
                mq[g] = fmaf(s, z, mn);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 Xg = *reinterpret_cast<const f32x4*>(xtab + ((int(j) * 4 + g) * 16 + 4 * qs));
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(mq[g], Xg[v], fmaf(sq[g], Dq[g][v], acc[v]));
            }
        } else if constexpr (Q4) {
            // x from memory: as above, with X = a second MFMA against ones,
            // group by group (four pending groups would not fit in
            // registers beside this variant's ring).
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x4 au = g == 0 ? it.a0 : g == 1 ? it.a1 : g == 2 ? it.a2 : it.a3;
                const bf16x8 a = __builtin_bit_cast(bf16x8, au);
                const float s = half_bits(it.m4[g]);
                const float mn = half_bits(it.m4[g] >> 16);
                const float t = -mn * __builtin_amdgcn_rcpf(s);
                // z = clamp(rint(-min / scale), 0, 15), branch-free; a NaN
                // ratio gives 0 (fmaxf returns the number).
                const float z = fminf(fmaxf(rintf(t), 0.0f), 15.0f);
                const float mp = fmaf(s, z, mn);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 Dg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a, widen_q4(it.c[g], __builtin_amdgcn_perm(0u, uint32_t(z), 0u)), zero, 0, 0, 0);
                const f32x4 Xg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(mp, Xg[v], fmaf(s, Dg[v], acc[v]));
            }
        } else {
            u32x4 a0u, a1u;
            if constexpr (XG) {
                a0u = it.a0;
                a1u = it.a1;
            } else {
                a0u = xs_row[int(j) * 8 + o0];
                a1u = xs_row[int(j) * 8 + o1];
            }
            const bf16x8 a0 = __builtin_bit_cast(bf16x8, a0u);
            const bf16x8 a1 = __builtin_bit_cast(bf16x8, a1u);
            const bf16x8 b0 = widen8(it.c.x, it.c.y);
            const bf16x8 b1 = widen8(it.c.z, it.c.w);
            if constexpr (FMT == FMT_Q8PC) {
                // One fp32 scale per row: the products of all the wave's
                // steps of the tile accumulate in D, scaled once at its end.
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, D, 0, 0, 0);
            } else {
                // A finished group's acc += s D waits until the next
                // group's MFMAs are issued, so the wave does not stall on
                // the MFMA result; the adds keep their order (the same bits).
                const bool opens = j % SPG == 0;
                if (opens) D = f32x4{0.f, 0.f, 0.f, 0.f};
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, D, 0, 0, 0);
                if (opens) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[v] = fmaf(s_done, D_done[v], acc[v]);
                }
                if (j % SPG == SPG - 1) {
                    D_done = D;
                    s_done = half_bits(it.s);
                }
            }
        }
        if (++j == j_hi) {
            if constexpr (FMT == FMT_Q8PC) {
                const float s = __uint_as_float(it.s);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = s * D[v];
                D = f32x4{0.f, 0.f, 0.f, 0.f};
            } else if constexpr (!Q4) {
                // The tile's last group; the next tile opens with a zero
                // pending group (0 * 0 added to a zero acc leaves +0).
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] = fmaf(s_done, D_done[v], acc[v]);
                D_done = f32x4{0.f, 0.f, 0.f, 0.f};
                s_done = 0.f;
            }
            if constexpr (KSPLIT == 1) {
                const int64_t row = tile * 16 + rho;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 4 * qs + v;
                    if (i < m && row < p.N) p.y[int64_t(i) * p.ldy + row] = acc[v];
                }
            } else {
                part[(buf * KSPLIT + wave) * 64 + lane] = acc;
                __syncthreads();
                // Thread t < 256 adds value t of the 16 x 16 output tile over
                // the parts, in K order.
                const int t = threadIdx.x;
                if (t < 256) {
                    const int L = t >> 2, v = t & 3;
                    float sum = part[(buf * KSPLIT) * 64 + L][v];
#pragma unroll
                    for (int w = 1; w < KSPLIT; ++w) sum += part[(buf * KSPLIT + w) * 64 + L][v];
                    const int i = 4 * (L >> 4) + v;
                    const int64_t row = tile * 16 + (L & 15);
                    if (i < m && row < p.N) p.y[int64_t(i) * p.ldy + row] = sum;
                }
                buf ^= 1;
            }
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            tile += W;
            j = j_lo;
        }
    };

    int64_t n = 0;
    for (; n + 2 * DEPTH <= n_items; n += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            consume(ring[d]);
            load(ring[d], ld);
            advance(ld);
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        if (n + d < n_items) {
            consume(ring[d]);
            if (n + DEPTH + d < n_items) {
                load(ring[d], ld);
                advance(ld);
            }
        }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (n + DEPTH + d < n_items) consume(ring[d]);
}

template <int FMT, int KSPLIT, bool XG>
hipError_t launch_fmt(const MmaParams& kp, int64_t waves, size_t lds, hipStream_t s)
{
    // Ring depth 8, or 6 with sixteen waves (a CU then has 96 KiB in
    // flight), or 4 when the ring also carries the A fragments.  Q4G32
    // items carry 16 bytes of meta per lane: 6, or 4 with sixteen waves,
    // or 3 with their four A fragments.
    constexpr int depth = XG ? (FMT == FMT_Q4G32 ? 3 : 4)
                        : FMT == FMT_Q4G32 ? (KSPLIT == 16 ? 4 : 6)
                                           : (KSPLIT == 16 ? 6 : 8);
    auto kern = qgemv_mma<FMT, depth, KSPLIT, XG>;
    static const hipError_t attr = [&] {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 int(kMaxDynLdsBytes));
        if (e != hipSuccess) (void)hipGetLastError();
        return e;
    }();
    if (attr != hipSuccess && lds > 64 * 1024) return attr;
    constexpr int threads = mma_threads<KSPLIT>();
    const int64_t wpg = threads / 64;
    const unsigned blocks = unsigned((waves + wpg - 1) / wpg);
    // Tile streams: one per wave, or one per work-group with a K split.
    MmaParams k = kp;
    const int64_t W = KSPLIT == 1 ? int64_t(blocks) * wpg : int64_t(blocks);
    k.tiles_q = kp.tiles / W;
    k.tiles_r = kp.tiles % W;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), lds, s, k);
    return hipGetLastError();
}

}  // namespace

namespace {
template <int FMT>
hipError_t launch_split(int ksplit, bool xg, const MmaParams& kp, int64_t waves, size_t lds, hipStream_t s)
{
    switch (ksplit * 2 + (xg ? 1 : 0)) {
    case 2: return launch_fmt<FMT, 1, false>(kp, waves, lds, s);
    case 3: return launch_fmt<FMT, 1, true>(kp, waves, lds, s);
    case 8: return launch_fmt<FMT, 4, false>(kp, waves, lds, s);
    case 9: return launch_fmt<FMT, 4, true>(kp, waves, lds, s);
    case 32: return launch_fmt<FMT, 16, false>(kp, waves, lds, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_mma(int fmt, int ksplit, bool xg, const MmaParams& kp, int64_t waves, size_t lds,
                      hipStream_t s)
{
    switch (fmt) {
    case FMT_Q8G64: return launch_split<FMT_Q8G64>(ksplit, xg, kp, waves, lds, s);
    case FMT_Q8G128: return launch_split<FMT_Q8G128>(ksplit, xg, kp, waves, lds, s);
    case FMT_Q8PC: return launch_split<FMT_Q8PC>(ksplit, xg, kp, waves, lds, s);
    case FMT_Q4G32: return launch_split<FMT_Q4G32>(ksplit, xg, kp, waves, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qg
