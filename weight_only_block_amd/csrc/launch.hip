// Host side of the launch: picks the wave count, ring depth and tile mapping
// for a matrix and calls the format's kernel (kern_*.hip).  No device code.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <string.h>

#include <atomic>
#include <mutex>

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

// Launch-geometry override (qg_set_launch_override), process-wide.  The
// three fields are packed into one atomic word, so a call made while
// another thread changes the override sees either the old or the new
// geometry, never a mix: target_waves in bits 0..39, contig + 1 in bits
// 40..41, shape + 1 in bits 42..44.
static std::atomic<uint64_t> g_override_word{(uint64_t(0) << 40) | (uint64_t(0) << 42)};

void set_launch_override(const LaunchOverride& o)
{
    const uint64_t w = (uint64_t(o.target_waves) & ((uint64_t(1) << 40) - 1)) |
                       (uint64_t(o.contig + 1) << 40) | (uint64_t(o.shape + 1) << 42);
    g_override_word.store(w, std::memory_order_relaxed);
}

static LaunchOverride current_override()
{
    const uint64_t w = g_override_word.load(std::memory_order_relaxed);
    LaunchOverride o;
    o.target_waves = int64_t(w & ((uint64_t(1) << 40) - 1));
    o.contig = int((w >> 40) & 3) - 1;
    o.shape = int((w >> 42) & 7) - 1;
    o.use_policy = 1;
    return o;
}

// QG_FORCE_VARIANT, read at every call (so that an A/B run and graph
// capture in one process pick up a change at the next call, as the per-call
// environment knobs of the vllm.cpp pull request #1936 commit log): a comma
// list of waves=<total waves>, wpcu=<waves per compute unit>, contig=0|1 and
// ring=2|4|xr (xr: x in registers, where the layout allows it) for the plain
// kernels, ksplit=1|4|16, xg=0|1, mmawaves=<waves>, mmacu=<work-groups
// per CU> and mmaeven=0|1 for the matrix-core kernel, optionally restricted to one shape with n=<N>, k=<K> and m=<m>
// (calls of other shapes are then not forced), and policy=0 to leave out the
// exact-shape policies below (for A/B runs of the policies themselves).
// Unknown keys and bad values are ignored; an unset or empty variable
// forces nothing.
static LaunchOverride forced_variant(int64_t cus, int64_t N, int64_t K, int m)
{
    LaunchOverride o;
    o.target_waves = 0;
    o.contig = -1;
    o.shape = -1;
    const char* e = getenv("QG_FORCE_VARIANT");
    if (!e) return o;
    bool other_shape = false;
    o.use_policy = 1;
    while (*e) {
        const char* eq = strchr(e, '=');
        if (!eq) break;
        const char* end = strchr(eq, ',');
        const size_t klen = size_t(eq - e);
        char* stop = nullptr;
        const long v = strtol(eq + 1, &stop, 10);
        const bool num = stop != eq + 1 && (stop == end || (!end && *stop == 0));
        if (klen == 5 && !strncmp(e, "waves", 5) && num && v > 0 && v <= (1L << 24)) o.target_waves = v;
        else if (klen == 4 && !strncmp(e, "wpcu", 4) && num && v > 0 && v <= 64) o.target_waves = v * cus;
        else if (klen == 6 && !strncmp(e, "contig", 6) && num && (v == 0 || v == 1)) o.contig = int(v);
        else if (klen == 1 && e[0] == 'n' && num && v != N) other_shape = true;
        else if (klen == 1 && e[0] == 'k' && num && v != K) other_shape = true;
        else if (klen == 1 && e[0] == 'm' && num && v != m) other_shape = true;
        else if (klen == 6 && !strncmp(e, "policy", 6) && num && (v == 0 || v == 1)) o.use_policy = int(v);
        else if (klen == 6 && !strncmp(e, "ksplit", 6) && num && (v == 1 || v == 4 || v == 16)) o.mma_ksplit = int(v);
        else if (klen == 2 && !strncmp(e, "xg", 2) && num && (v == 0 || v == 1)) o.mma_xg = int(v);
        else if (klen == 8 && !strncmp(e, "mmawaves", 8) && num && v > 0 && v <= (1L << 24)) o.mma_waves = v;
        else if (klen == 5 && !strncmp(e, "mmacu", 5) && num && v >= 1 && v <= 8) o.mma_per_cu = int(v);
        else if (klen == 7 && !strncmp(e, "mmaeven", 7) && num && (v == 0 || v == 1)) o.mma_even = int(v);
        else if (klen == 4 && !strncmp(e, "ring", 4)) {
            if (num && v == 2) o.shape = SHAPE_D2_W4;
            else if (num && v == 4) o.shape = SHAPE_D4_W4;
            else if (!strncmp(eq + 1, "xr", 2) && (eq[3] == ',' || eq[3] == 0)) o.shape = SHAPE_XR;
        }
        if (!end) break;
        e = end + 1;
    }
    if (other_shape) {
        LaunchOverride none;
        none.target_waves = 0;
        none.contig = -1;
        none.shape = -1;
        return none;
    }
    return o;
}

// Exact-shape launch policy: geometries that measured faster than the
// defaults below for one (format, m, N, K, grouped) shape, each admitted by
// interleaved A/B pairs (the evidence is recorded with the measurements);
// every other shape takes the defaults.  This is the per-shape, measured
// operator policy of the MetaInfer-cpp README (milestone M6.5-E,
// MeasuredOperatorPolicy), for launch geometry.
// Policy key of the grouped gate/up calls with the SwiGLU epilogue (their
// pair layout is a Q4G32 layout; they are keyed apart from plain grouped
// Q4G32 calls, with N = the gate rows).
constexpr int kPolicySwiglu = 5;

struct ShapePolicy {
    int fmt, m;
    int64_t N, K;
    bool grouped;
    int64_t waves_per_cu;   // 0: default
    int contig;             // -1: default
    int shape;              // -1: default
};
// Entries were admitted on MI355X by interleaved pairs in one process
// (bench.py --sweep, 500 steps per arm, five pairs): at least 4 of 5 pairs
// won and a median gain of at least 0.5%.  Medians are us per step of the
// workload the shape belongs to, default -> entry.
static const ShapePolicy kPolicy[] = {
    // Q4G32 K=2560 family, m = 1: ring 2 + contiguous 21.45 -> 20.36 (5/5)
    {FMT_Q4G32, 1, 9216, 2560, false, 0, 1, SHAPE_D2_W4},
    // contiguous 21.44 -> 21.20 (5/5)
    {FMT_Q4G32, 1, 2560, 9216, false, 0, 1, -1},
    // m = 4: ring 2 34.60 -> 34.22 (5/5)
    {FMT_Q4G32, 4, 9216, 2560, false, 0, -1, SHAPE_D2_W4},
    // Qwen3-14B TP4 W8A16 layer, m = 1: contiguous 37.69 -> 37.50 (5/5)
    {FMT_Q8PC, 1, 1792, 5120, false, 0, 1, -1},
    // contiguous 37.67 -> 37.48 (5/5)
    {FMT_Q8PC, 1, 5120, 1280, false, 0, 1, -1},
    // x in registers + contiguous 37.74 -> 37.49 (5/5)
    {FMT_Q8PC, 1, 8704, 5120, false, 0, 1, SHAPE_XR},
    // contiguous 37.71 -> 37.58 (5/5)
    {FMT_Q8PC, 1, 5120, 4352, false, 0, 1, -1},
    // m = 4: ring 2 53.80 -> 53.40 (5/5) and 53.80 -> 52.50 (5/5)
    {FMT_Q8PC, 4, 1792, 5120, false, 0, -1, SHAPE_D2_W4},
    {FMT_Q8PC, 4, 8704, 5120, false, 0, -1, SHAPE_D2_W4},
    // Qwen3-0.6B-shaped layer: x in registers 30.55 -> 30.35 (4/5),
    // ring 2 30.33 -> 30.13 (4/5), x in registers 30.38 -> 30.19 (4/5);
    // the 1024 x 1024 matrices (k, v, and the Q8G64 N = K = 1024 GEMV)
    // ring 2: layer 25.23 -> 24.38 (5/5, graph replay), the single GEMV
    // 3.95 -> 3.55 (graph) and 3.94 -> 3.64 (eager, 5/5 each)
    {FMT_Q8G64, 1, 1024, 1024, false, 0, -1, SHAPE_D2_W4},
    // Projections stacked into one launch (q+k+v and gate+up sharing an
    // activation): the 0.6B layer's gate+up 6144 x 1024, x in registers,
    // stacked layer 16.08 -> 15.37 (4/5, graph replay), then contiguous
    // 15.36 -> 15.20 (5/5); the Q4G32 K=2560 family's gate+up 18432 x 2560,
    // x in registers, 17.06 -> 16.09 (5/5)
    {FMT_Q8G64, 1, 6144, 1024, false, 0, 1, SHAPE_XR},
    {FMT_Q4G32, 1, 18432, 2560, false, 0, -1, SHAPE_XR},
    {FMT_Q8G64, 1, 1024, 2048, false, 0, -1, SHAPE_XR},
    {FMT_Q8G64, 1, 3072, 1024, false, 0, -1, SHAPE_D2_W4},
    {FMT_Q8G64, 1, 1024, 3072, false, 0, -1, SHAPE_XR},
    // Routed experts (8 of 128): x in registers, three-call flow 24.50 ->
    // 24.02 (gate/up, 5/5) and 24.45 -> 24.19 (down, 5/5); merged flow
    // (down) 20.80 -> 20.58 (5/5), merged gate+up 20.75 -> 20.62 (4/5)
    {FMT_Q4G32, 1, 1536, 4096, true, 0, -1, SHAPE_XR},
    {FMT_Q4G32, 1, 4096, 1536, true, 0, -1, SHAPE_XR},
    {FMT_Q4G32, 1, 3072, 4096, true, 0, -1, SHAPE_XR},
    // Routed gate/up with the SwiGLU epilogue: x in registers, fused flow
    // 20.76 -> 20.62 (5/5)
    {kPolicySwiglu, 1, 1536, 4096, true, 0, -1, SHAPE_XR},
    {-1, 0, 0, 0, false, 0, -1, -1},   // (end)
};

static const ShapePolicy* policy_for(int fmt, int m, int64_t N, int64_t K, bool grouped)
{
    for (const ShapePolicy& e : kPolicy) {
        if (e.fmt < 0) break;
        if (e.fmt == fmt && e.m == m && e.N == N && e.K == K && e.grouped == grouped) return &e;
    }
    return nullptr;
}

// Per-wave timeline (qg_set_wave_trace): a caller buffer of records, filled
// launch after launch until it is full; later launches go untraced and are
// counted as dropped.  The flag keeps the untraced path to one relaxed load.
static std::mutex g_trace_mu;
static std::atomic<bool> g_trace_on{false};
static unsigned long long* g_trace_buf = nullptr;
static int64_t g_trace_cap = 0, g_trace_used = 0, g_trace_launches = 0, g_trace_dropped = 0;

void set_wave_trace(void* buf, int64_t capacity)
{
    std::lock_guard<std::mutex> lock(g_trace_mu);
    g_trace_buf = static_cast<unsigned long long*>(buf);
    g_trace_cap = buf ? capacity : 0;
    g_trace_used = g_trace_launches = g_trace_dropped = 0;
    g_trace_on.store(buf != nullptr, std::memory_order_relaxed);
}

void wave_trace_state(int64_t* records, int64_t* launches, int64_t* dropped)
{
    std::lock_guard<std::mutex> lock(g_trace_mu);
    *records = g_trace_used;
    *launches = g_trace_launches;
    *dropped = g_trace_dropped;
}

unsigned long long* reserve_wave_trace(int64_t waves, int64_t* launch_index)
{
    *launch_index = 0;
    if (!g_trace_on.load(std::memory_order_relaxed)) return nullptr;
    std::lock_guard<std::mutex> lock(g_trace_mu);
    if (!g_trace_buf) return nullptr;
    if (waves > g_trace_cap - g_trace_used) {
        ++g_trace_dropped;
        return nullptr;
    }
    unsigned long long* r = g_trace_buf + g_trace_used * 8;
    g_trace_used += waves;
    *launch_index = g_trace_launches++;
    return r;
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
    kp.trace = nullptr;
    kp.trace_launch = 0;
    kp.inv_U = 1.0f / float(L.U);
    const int slots = a.grouped ? a.n_slots : 1;
    // Geometry, first match wins: qg_set_launch_override, QG_FORCE_VARIANT,
    // the exact-shape policy, then the defaults.
    const int64_t cus = compute_units();
    const LaunchOverride api = current_override();
    const LaunchOverride env = forced_variant(cus, a.swiglu ? a.n_out : L.N, L.K, a.m);
    // The swiglu pair layout is a Q4G32 layout of Nv rows; its shapes are
    // looked up with N = the gate rows, as the call names them.
    const ShapePolicy* pol =
        env.use_policy ? policy_for(a.swiglu ? kPolicySwiglu : L.fmt, a.m, a.swiglu ? a.n_out : L.N, L.K,
                                    a.grouped)
                       : nullptr;
    // About target_waves waves in total, never more waves than tiles; k
    // tiles per wave, then the fewest waves that cover the tiles with k
    // each, so all waves get k tiles (a few k-1), never k for some and k/2
    // for others.
    int64_t target_waves =
        cus * (a.grouped ? kWavesPerCuGrouped : (a.m > 1 ? kWavesPerCuDenseMulti : kWavesPerCuDense));
    if (pol && pol->waves_per_cu > 0) target_waves = cus * pol->waves_per_cu;
    if (env.target_waves > 0) target_waves = env.target_waves;
    if (api.target_waves > 0) target_waves = api.target_waves;
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
    // keep the grid-stride window.
    bool contig = a.grouped;
    if (pol && pol->contig >= 0) contig = pol->contig != 0;
    if (env.contig >= 0) contig = env.contig != 0;
    if (api.contig >= 0) contig = api.contig != 0;
    kp.contig_k = contig ? k : 0;
    if (pol && pol->shape >= 0) shape = pol->shape;
    if (env.shape >= 0) shape = env.shape;
    if (api.shape >= 0) shape = api.shape;
    // x in registers only where the kernel is built for the layout (and not
    // with the argmax epilogue, whose tail shares LDS); elsewhere a request
    // for it keeps the staged kernel with the default ring.
    if (shape == SHAPE_XR && (!xr_supported(L, a.m) || a.argmax))
        shape = (L.J <= 3 && k >= 2) ? SHAPE_D2_W4 : SHAPE_D4_W4;
    kp.x_vec16 = ((reinterpret_cast<uintptr_t>(a.x) | uintptr_t(a.ldx * 2) |
                   uintptr_t(a.x_slot_stride * 2)) & 15u) == 0;
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

// Exact-shape policy of the matrix-core kernel's launch, admitted like
// kPolicy above (interleaved pairs, at least 4 of 5 won, median gain of at
// least 0.5%; medians are us per step of the Qwen3-14B TP4 W8A16 layer, or
// of the Q4G32 K=2560 family, on the matrix cores, default -> entry).
// per_cu: work-groups per CU (0: default); even: when the tiles outnumber
// the resident work-groups, the fewest work-groups that give every one the
// same number of tiles, so that no round runs part-empty; ksplit (1, 4 or
// 16) and xg (0: x staged, 1: x read from memory) as the keys of
// QG_FORCE_VARIANT (-1: the default choice).
struct MmaShapePolicy {
    int fmt, m_lo, m_hi;   // the entry covers m_lo <= m <= m_hi
    int64_t N, K;
    int per_cu;
    bool even;
    int ksplit;
    int xg;
};
static const MmaShapePolicy kMmaPolicy[] = {
    // gate/up 5120 -> 8704, m = 4: even rounds 48.03 -> 46.57 (5/5); after
    // the per-tile Q8PC scaling, m = 2 45.69 -> 44.00, m = 3 45.71 -> 44.07
    // (5/5 each)
    {FMT_Q8PC, 2, 4, 8704, 5120, 0, true, -1, -1},
    // down 4352 -> 5120, m = 4: even rounds 48.05 -> 47.70 (5/5); m = 2
    // 45.69 -> 45.37, m = 3 45.75 -> 45.45 (5/5 each)
    {FMT_Q8PC, 2, 4, 5120, 4352, 0, true, -1, -1},
    // gate/up, m = 8: even rounds 49.14 -> 47.81 (5/5)
    {FMT_Q8PC, 8, 8, 8704, 5120, 0, true, -1, -1},
    // o 1280 -> 5120: a four-way K split with x read from memory, m = 4
    // 43.86 -> 42.87, m = 8 45.47 -> 44.61, m = 16 75.02 -> 74.38; m = 2
    // 45.70 -> 44.70, m = 3 45.73 -> 44.75 (5/5 each)
    {FMT_Q8PC, 2, 4, 5120, 1280, 0, false, 4, 1},
    {FMT_Q8PC, 8, 8, 5120, 1280, 0, false, 4, 1},
    {FMT_Q8PC, 16, 16, 5120, 1280, 0, false, 4, 1},
    // Q4G32 gate/up 2560 -> 9216, m = 16: a four-way K split with x read
    // from memory, three-GEMV step 47.38 -> 45.90 (5/5; it had taken a
    // sixteen-way split, 58.86 -> 51.23, before the per-group sums moved
    // into an LDS table)
    {FMT_Q4G32, 16, 16, 9216, 2560, 0, false, 4, 1},
    {-1, 0, 0, 0, 0, 0, false, -1, -1},   // (end)
};

static const MmaShapePolicy* mma_policy_for(int fmt, int m, int64_t N, int64_t K)
{
    for (const MmaShapePolicy& e : kMmaPolicy) {
        if (e.fmt < 0) break;
        if (e.fmt == fmt && e.m_lo <= m && m <= e.m_hi && e.N == N && e.K == K) return &e;
    }
    return nullptr;
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
    // QG_FORCE_VARIANT's ksplit=1|4|16 forces the split, xg=0|1 the x path
    // and mmawaves the wave count the choice is made for (tuning sweeps).
    const LaunchOverride env = forced_variant(compute_units(), kp.N, kp.K, kp.m);
    // QG_FORCE_VARIANT's policy=0 leaves the shape policy out here too.
    const MmaShapePolicy* pol = env.use_policy ? mma_policy_for(fmt, kp.m, kp.N, kp.K) : nullptr;
    const int64_t env_waves = env.mma_waves;
    // The forced K split and x path, else the policy's, else the defaults.
    const int env_split = env.mma_ksplit > 0 ? env.mma_ksplit : (pol ? pol->ksplit : -1);
    const int env_xg = env.mma_xg >= 0 ? env.mma_xg : (pol ? pol->xg : -1);
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
    // xg=0/1 forces staging on (where x fits) / x from memory.
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
        int64_t most = split == 16 ? 1 : 2;
        if (pol && pol->per_cu > 0 && split != 16) most = pol->per_cu;
        if (env.mma_per_cu > 0 && split != 16) most = env.mma_per_cu;
        per_cu = per_cu < 1 ? 1 : (per_cu > most ? most : per_cu);
        const int64_t resident = compute_units() * per_cu;
        int64_t wgs = kp.tiles < resident ? kp.tiles : resident;
        const bool even = env.mma_even >= 0 ? env.mma_even == 1 : (pol && pol->even);
        if (even && kp.tiles > resident) {
            const int64_t rounds = (kp.tiles + resident - 1) / resident;
            wgs = (kp.tiles + rounds - 1) / rounds;
        }
        return launch_mma(fmt, split, xg, kp, wgs * split, per_wg, s);
    }
    const int64_t k = (kp.tiles + cap - 1) / cap;
    const int64_t waves = (kp.tiles + k - 1) / k;
    return launch_mma(fmt, 1, xg, kp, waves, xg ? 0 : lds, s);
}

}  // namespace qg
