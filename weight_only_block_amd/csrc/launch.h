// Internal interface between the C ABI (abi.cpp) and the kernels
// (kern_*.hip).  Not installed; callers use include/qgemv.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace qg {

// LDS a work-group may use on gfx950, and the part of it left for the
// dynamic (activation) area once 1 KiB is set aside for the kernels' own
// static LDS (the argmax epilogue's per-wave keys).
constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr size_t kMaxDynLdsBytes = kMaxLdsBytes - 1024;

// Kernel arguments (passed by value).
struct KernelParams {
    const uint8_t* w;          // packed matrix; grouped: expert 0
    int64_t expert_stride;     // bytes between packed experts
    const int32_t* ids;        // device expert id per slot (grouped)
    int32_t n_experts;
    int32_t N;
    int32_t K;
    const uint16_t* x;         // bf16 activations
    int64_t ldx;               // elements between activation rows
    int64_t x_slot_stride;     // elements between slot activations
    float* y;
    int64_t ldy;               // elements between output rows
    int64_t y_slot_stride;     // elements between slot outputs
    int64_t J;                 // steps per tile
    int64_t tiles;
    int64_t tiles_q, tiles_r;  // grid-stride mapping: tiles = tiles_q * waves + tiles_r
    int64_t code_bytes;        // offset of the meta blocks
    int64_t meta_step_bytes;
    int64_t meta_tile_bytes;   // per-tile meta after the steps' meta (Q8PC row scales)
    int64_t contig_k;          // > 0: each wave streams contig_k consecutive tiles
    uint16_t* act;             // SwiGLU epilogue: bf16 output per slot
    int64_t act_slot_stride;   // elements between slot outputs (SwiGLU)
    int32_t n_out;             // outputs per slot (SwiGLU: gate rows)
    int32_t* idx_out;          // argmax epilogue: chosen index per activation row
    unsigned long long* keys;  // argmax epilogue: one key per row (zero between calls)
    unsigned int* counter;     // argmax epilogue: finished work-groups (zero between calls)
    float cert_t;              // Q4G32: certificate threshold T (q4_cert_threshold)
    int32_t x_vec16;           // x in registers: x, ldx and x_slot_stride allow 16-byte loads
    float inv_U;               // 1.0f / (units per row), for the staging's row index
    unsigned long long* trace; // per-wave timeline records of this launch (null: off)
    int64_t trace_launch;      // the launch's index in the timeline
};

// Per-wave timeline (qg_set_wave_trace): reserves the records of a launch of
// `waves` waves and returns where they go, or null when tracing is off or
// the buffer is full.  Host code.
unsigned long long* reserve_wave_trace(int64_t waves, int64_t* launch_index);

// Threshold T of the Q4G32 fast path's certificate (kernel_body.h,
// kQ4Kappa): a row's fast sum is accepted when
//     C = sum_g (T |y_g| - kappa (|s| + |min| / 256) XA_g) >= 0.
// The bar is |y - y_exact| <= 2e-3 * sum |w x|; sum |w x| >= A - kappa E
// with A = sum |y_g| and E the sum of the kappa terms' factors, and adding
// the J per-lane partial sums and the log2(64) reduction levels costs at
// most (J + 7) * 2^-24 * A more (the same for forming A).  So kappa E +
// (J + 7) u A <= 2e-3 (A (1 - (J + 7) u) - kappa E) is enough, which holds
// when kappa E <= A (2e-3 - 2.01 (J + 7) u) / 1.002.  C itself is summed in
// fp32 over the same J + 7 steps, so T is reduced by a further relative
// 4 (J + 7) u, and by 1e-6 for the rounding of each term.
inline float q4_cert_threshold(int64_t J)
{
    const double u = 1.0 / 16777216.0;
    const double t = (2e-3 - 2.01 * double(J + 7) * u) / 1.002;
    return float(t * (1.0 - 4.0 * double(J + 7) * u) - 1e-6);
}

// Launch shape: ring depth 2 or 4 items with x staged in LDS; or x held in
// registers with a ring of one tile (J = 2, 3 or 5 steps, m = 1, G >= 16).
// Work-groups are 4 waves.
enum Shape { SHAPE_D2_W4 = 0, SHAPE_D4_W4 = 1, SHAPE_XR = 2 };

// Whether a layout can take the x-in-registers kernel (m activation rows).
inline bool xr_supported(const Layout& L, int m)
{
    return m == 1 && L.G >= 16 && (L.J == 2 || L.J == 3 || L.J == 5);
}

struct LaunchArgs {
    Layout layout;
    bool grouped;
    int m;
    const void* w;
    int64_t expert_stride;
    const int32_t* ids;
    int32_t n_experts;
    int32_t n_slots;
    const uint16_t* x;
    int64_t ldx;
    int64_t x_slot_stride;
    float* y;
    int64_t ldy;
    int64_t y_slot_stride;
    bool swiglu;               // gate/up pair layout with the SwiGLU epilogue
    uint16_t* act;
    int64_t act_slot_stride;
    int64_t n_out;
    bool argmax;               // argmax epilogue (dense Q8G64 / Q8G128)
    int32_t* idx_out;
    void* argmax_workspace;    // keys[m], then the counter
    hipStream_t stream;
};

// Process-wide launch-geometry override of the VALU kernels (tests and
// tuning sweeps; the results are the same bits for every geometry).
struct LaunchOverride {
    int64_t target_waves;  // > 0: about this many waves in total
    int contig;            // 1: contiguous tile runs per wave, 0: grid-stride, -1: default
    int shape;             // SHAPE_D2_W4 / SHAPE_D4_W4 / SHAPE_XR, -1: default
    int use_policy = 1;    // 0: leave out the exact-shape policy (QG_FORCE_VARIANT only)
    // Matrix-core kernel (QG_FORCE_VARIANT only): K split 1, 4 or 16 (-1:
    // default), x read from memory (1) or staged (0) (-1: default), and the
    // wave count that decides whether to split (0: default).
    int mma_ksplit = -1;
    int mma_xg = -1;
    int64_t mma_waves = 0;
    // Split launches: work-groups per CU (0: default) and even rounds (1 on,
    // 0 off, -1: default).
    int mma_per_cu = 0;
    int mma_even = -1;
};
void set_launch_override(const LaunchOverride& o);
void set_wave_trace(void* buf, int64_t capacity);
void wave_trace_state(int64_t* records, int64_t* launches, int64_t* dropped);

// Bytes of dynamic LDS a launch of this layout needs for m activation rows.
size_t lds_bytes_for(const Layout& L, int m);

// Enqueues the kernel; returns the HIP status of the launch.
hipError_t launch(const LaunchArgs& a);

// Per-format kernel launchers (kern_<format>.hip): m activation rows, lane
// group G, launch shape, waves per slot, slots (grid y), dynamic LDS bytes.
#define QG_DECLARE_LAUNCHER(name)                                                            \
    hipError_t name(int m, bool grouped, int G, int shape, const KernelParams& kp,            \
                    int64_t waves, int slots, size_t lds, hipStream_t s)
QG_DECLARE_LAUNCHER(launch_q8g64);
QG_DECLARE_LAUNCHER(launch_q4g32);
QG_DECLARE_LAUNCHER(launch_q8g128);
QG_DECLARE_LAUNCHER(launch_q8pc);
#undef QG_DECLARE_LAUNCHER
// Matrix-core kernel (kern_mma.hip): 8-bit formats in the MmaLayout,
// m = 2..16 activation rows.
struct MmaParams {
    const uint8_t* w;
    const uint16_t* x;
    float* y;
    int64_t ldx, ldy;
    int32_t m;
    int32_t N;
    int64_t K, J, tiles, code_bytes, meta_tile_bytes;
    int64_t tiles_q, tiles_r;  // tiles = tiles_q * W + tiles_r for the launch's W tile streams
    float inv_cpr;             // 1.0f / (16-byte chunks per activation row), for the staging
};
// ksplit: 1 (each wave streams whole tiles), 4 or 16 (the waves of a
// work-group share each tile's K).  xg (with ksplit 4): x is read from
// memory with each item instead of staged in LDS.
hipError_t launch_mma(int fmt, int ksplit, bool xg, const MmaParams& kp, int64_t waves, size_t lds,
                      hipStream_t s);
// LDS a K split adds after the staged activations: two buffers of
// ksplit waves x 64 lanes x 4 floats.
constexpr size_t mma_split_lds_bytes(int ksplit)
{
    return size_t(2) * ksplit * 64 * 16;
}
// Picks the wave count for the matrix-core kernel and launches it.
hipError_t launch_mma_sized(int fmt, const MmaParams& kp, size_t lds, hipStream_t s);

// Dense Q8G64 / Q8G128 with the argmax epilogue (kern_argmax_epi.hip).
hipError_t launch_argmax_epilogue(int fmt, int m, int G, int shape, const KernelParams& kp,
                                  int64_t waves, size_t lds, hipStream_t s);
// Grouped Q4G32 with the SwiGLU epilogue (kern_q4g32_swiglu.hip), m = 1.
hipError_t launch_q4g32_swiglu(int G, int shape, const KernelParams& kp, int64_t waves, int slots,
                               size_t lds, hipStream_t s);

}  // namespace qg
