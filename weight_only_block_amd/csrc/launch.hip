// Host side of the launch: picks the wave count, ring depth and tile mapping
// for a matrix and calls the format's kernel (kern_*.hip).  No device code.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "launch.h"

namespace qg {

namespace {
// Wave counts are per compute unit: a dense sweep at m = 1 runs one 4-wave
// work-group per CU (every CU streams the same bytes and the launch reads
// one window of about CUs*4 tiles at a time); at m >= 2, where each byte
// costs more VALU work, two work-groups per CU hide more of it (LM head at
// m = 4: 90 -> 79 us); routed-expert launches run two.  All measured best on
// MI355X; at m = 1, two work-groups per CU measured 7% slower.
constexpr int64_t kWavesPerCuDense = 4;
constexpr int64_t kWavesPerCuDenseMulti = 8;
constexpr int64_t kWavesPerCuGrouped = 8;
}  // namespace

// Launch-geometry override (qg_set_launch_override): 0 / -1 leave the
// choice to the environment (QG_TARGET_WAVES, QG_CONTIG, QG_SHAPE, read once,
// for tuning sweeps) and then to the defaults below.
static LaunchOverride g_override = {0, -1, -1};

void set_launch_override(const LaunchOverride& o)
{
    g_override = o;
}

// Compute units of the current device, looked up once per device.
static int64_t compute_units()
{
    // Calls may come from several host threads: the cache is atomic (every
    // thread that finds it empty stores the same value).
    static std::atomic<int64_t> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int64_t v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        v = n;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

size_t lds_bytes_for(const Layout& L, int m)
{
    // The bf16 rows of x, plus two fp32 activation sums (sum x, sum |x|)
    // per 32-group for Q4G32 (the 8-bit formats need none).
    const int64_t sums = L.fmt == FMT_Q4G32 ? 2 * L.U : 0;
    return size_t(m) * size_t(L.K / 2 + sums) * 4;
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
    kp.meta_tile_bytes = L.meta_tile_bytes;
    kp.act = a.act;
    kp.act_slot_stride = a.act_slot_stride;
    kp.n_out = int32_t(a.n_out);
    kp.idx_out = a.idx_out;
    kp.keys = static_cast<unsigned long long*>(a.argmax_workspace);
    kp.counter = a.argmax_workspace ? reinterpret_cast<unsigned int*>(kp.keys + a.m) : nullptr;
    kp.cert_t = q4_cert_threshold(L.J);
    const int slots = a.grouped ? a.n_slots : 1;
    // About target_waves waves in total (QG_TARGET_WAVES overrides it, for
    // tuning sweeps), never more waves than tiles; k tiles per wave, then the
    // fewest waves that cover the tiles with k each, so all waves get k tiles
    // (a few k-1), never k for some and k/2 for others.
    static const int64_t env_waves = [] {
        const char* e = getenv("QG_TARGET_WAVES");
        const long v = e ? strtol(e, nullptr, 10) : 0;
        return v > 0 ? int64_t(v) : int64_t(0);
    }();
    const int64_t cus = compute_units();
    const int64_t target_waves =
        g_override.target_waves > 0 ? g_override.target_waves
        : env_waves                 ? env_waves
                                    : cus * (a.grouped ? kWavesPerCuGrouped
                                                       : (a.m > 1 ? kWavesPerCuDenseMulti : kWavesPerCuDense));
    int64_t cap = target_waves / slots;
    if (cap < 1) cap = 1;
    // Up to twice the cap, a dense launch is latency-bound rather than
    // stream-bound: one tile per wave gives it the most parallelism.
    const int64_t k = (!a.grouped && L.tiles <= 2 * cap) ? 1 : (L.tiles + cap - 1) / cap;
    const int64_t waves_per_slot = (L.tiles + k - 1) / k;
    // A ring of 2 only when the wave streams several shallow tiles; with a
    // single tile per wave the whole tile goes in flight at once.
    int shape = (L.J <= 3 && k >= 2) ? SHAPE_D2_W4 : SHAPE_D4_W4;
    // Routed-expert launches give each wave a contiguous run of k tiles (the
    // whole 31.5 MB call is in flight at once anyway, so a common window
    // buys nothing, and adjacent tiles measured ~3% faster); dense sweeps
    // keep the grid-stride window.  QG_CONTIG=0/1 overrides (tuning sweeps).
    static const int env_contig = [] {
        const char* e = getenv("QG_CONTIG");
        return e ? int(strtol(e, nullptr, 10)) : -1;
    }();
    const bool contig = g_override.contig >= 0 ? g_override.contig != 0
                      : env_contig >= 0         ? env_contig != 0
                                                : a.grouped;
    kp.contig_k = contig ? k : 0;
    static const int env_shape = [] {
        const char* e = getenv("QG_SHAPE");   // tuning sweeps only
        return e ? int(strtol(e, nullptr, 10)) : -1;
    }();
    if (env_shape == SHAPE_D2_W4 || env_shape == SHAPE_D4_W4) shape = env_shape;
    if (g_override.shape == SHAPE_D2_W4 || g_override.shape == SHAPE_D4_W4) shape = g_override.shape;
    const size_t lds = lds_bytes_for(L, a.m);
    const hipStream_t s = a.stream;
    const int64_t w = waves_per_slot;
    if (a.swiglu) return launch_q4g32_swiglu(L.G, shape, kp, w, slots, lds, s);
    if (a.argmax) return launch_argmax_epilogue(L.fmt, a.m, L.G, shape, kp, w, lds, s);
    switch (L.fmt) {
    case FMT_Q8G64: return launch_q8g64(a.m, a.grouped, L.G, shape, kp, w, slots, lds, s);
    case FMT_Q4G32: return launch_q4g32(a.m, a.grouped, L.G, shape, kp, w, slots, lds, s);
    case FMT_Q8G128: return launch_q8g128(a.m, a.grouped, L.G, shape, kp, w, slots, lds, s);
    case FMT_Q8PC: return launch_q8pc(a.m, a.grouped, L.G, shape, kp, w, slots, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mma_sized(int fmt, const MmaParams& kp, size_t lds, hipStream_t s)
{
    // Two 4-wave work-groups per CU.  With at least two tiles per wave the
    // waves stream whole tiles on their own (k tiles each, the fewest waves
    // that cover the tiles with k each); with fewer, the waves of a
    // work-group split each tile's K: sixteen of them where the row has at
    // least 64 scale groups and the LDS allows, else four (with fewer
    // groups per wave the per-tile fold outweighs the wider stream:
    // 5120 x 1280 Q8PC at m = 8 measured 6.3 us with four, 7.5 with sixteen).
    // QG_MMA_KSPLIT = 1, 4 or 16 forces the split (tuning sweeps).
    static const int64_t env_waves = [] {
        const char* e = getenv("QG_MMA_WAVES");   // tuning sweeps only
        const long v = e ? strtol(e, nullptr, 10) : 0;
        return v > 0 ? int64_t(v) : int64_t(0);
    }();
    static const int env_split = [] {
        const char* e = getenv("QG_MMA_KSPLIT");
        return e ? int(strtol(e, nullptr, 10)) : -1;
    }();
    static const int env_xg = [] {
        const char* e = getenv("QG_MMA_XG");        // tuning sweeps only
        return e ? int(strtol(e, nullptr, 10)) : -1;
    }();
    const int64_t cap = env_waves ? env_waves : compute_units() * 8;
    const int64_t groups_per_row = fmt == FMT_Q8G128 ? kp.J / 2 : kp.J;
    int split = (kp.tiles < 2 * cap && groups_per_row >= 4) ? 4 : 1;
    if (split == 4 && groups_per_row >= 64) split = 16;
    if ((env_split == 4 && groups_per_row >= 4) || (env_split == 16 && groups_per_row >= 16) || env_split == 1)
        split = env_split;
    // Where the sixteen-way split's partial sums do not fit beside the
    // staged x, four waves share the tile; where the staged x would leave
    // room for only one such group per CU, they read x from memory with
    // each item instead (two groups per CU; Q8PC at m = 15 measured 15.0 ->
    // 11.1 us on 1792 x 5120 and 17.2 -> 13.6 us on 5120 x 4352).  Q4G32
    // keeps staging as long as x fits.  Without a split, x is read from
    // memory only when it does not fit in LDS at all.
    // QG_MMA_XG = 0/1 forces staging on (where x fits) / x from memory.
    bool xg = false;
    if (split == 16 && lds + mma_split_lds_bytes(16) > kMaxDynLdsBytes) split = 4;
    if (split == 4) {
        const size_t staged = lds + mma_split_lds_bytes(4);
        xg = staged > kMaxDynLdsBytes || (fmt != FMT_Q4G32 && staged > kMaxLdsBytes / 2);
        if (env_xg == 0 && staged <= kMaxDynLdsBytes) xg = false;
    }
    if (split == 1) xg = lds > kMaxDynLdsBytes;
    if (split > 1 && env_xg == 1) {
        split = 4;
        xg = true;
    }
    if (split > 1) {
        // As many work-groups as can be resident at once (staged x bounds
        // how many fit in a CU's LDS; a 16-wave group takes a CU's share of
        // waves), each looping over its tiles: more than that would run in
        // uneven rounds.
        const size_t per_wg = (xg ? 0 : lds) + mma_split_lds_bytes(split);
        int64_t per_cu = int64_t(kMaxLdsBytes / per_wg);
        const int64_t most = split == 16 ? 1 : 2;
        per_cu = per_cu < 1 ? 1 : (per_cu > most ? most : per_cu);
        const int64_t resident = compute_units() * per_cu;
        const int64_t wgs = kp.tiles < resident ? kp.tiles : resident;
        return launch_mma(fmt, split, xg, kp, wgs * split, per_wg, s);
    }
    const int64_t k = (kp.tiles + cap - 1) / cap;
    const int64_t waves = (kp.tiles + k - 1) / k;
    return launch_mma(fmt, 1, xg, kp, waves, xg ? 0 : lds, s);
}

}  // namespace qg
