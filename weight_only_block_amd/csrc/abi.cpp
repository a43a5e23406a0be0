// C ABI of the decode GEMV library: argument validation on the host, the
// variant choice, and one kernel launch on the caller's stream.  Nothing
// here allocates or synchronizes.  Returning a status for every rejected
// request instead of falling back to another path follows the Qwen3 C++
// Reference Runtime README (its HIP backend reports Unsupported rather than
// silently running elsewhere); gating the number of activation rows on the
// GEMV itself follows the m-gate fix in the commit log of vllm.cpp pull
// request #1936, where a GEMV that only wrote row 0 was reached with m > 1.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/qgemv.h"
#include "argmax.h"
#include "launch.h"
#include "read_stream.h"

namespace {

// Route counters: one per (kind, m, log2 G).  kind 0 Q8G64, 1 Q4G32,
// 2 grouped Q4G32, 3 Q8G128, 4 Q8PC, 5 grouped Q4G32 with SwiGLU,
// 6 Q8G64 with the argmax epilogue, 7 Q8G128 with the argmax epilogue,
// 8..10 the matrix-core kernel for Q8G64, Q8G128, Q8PC, 11 the matrix-core
// kernel for Q4G32 (m up to 16; one shape per format, counted in the first
// G slot).
constexpr int kKinds = 12, kMs = 16, kGs = 7;
std::atomic<uint64_t> g_route[kKinds][kMs][kGs];

int log2i(int v)
{
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

const char* kind_name(int kind)
{
    switch (kind) {
    case 0: return "q8g64";
    case 1: return "q4g32";
    case 2: return "q4g32_grouped";
    case 3: return "q8g128";
    case 4: return "q8pc";
    case 5: return "q4g32_grouped_swiglu";
    case 6: return "q8g64_argmax";
    case 7: return "q8g128_argmax";
    case 8: return "q8g64_mma";
    case 9: return "q8g128_mma";
    case 10: return "q8pc_mma";
    default: return "q4g32_mma";
    }
}

// Route-counter kind of a dense format.
int kind_of(int fmt)
{
    switch (fmt) {
    case qg::FMT_Q8G64: return 0;
    case qg::FMT_Q4G32: return 1;
    case qg::FMT_Q8G128: return 3;
    default: return 4;
    }
}

void format_variant(int kind, int m, int G, char* buf, size_t len)
{
    if (kind >= 8) snprintf(buf, len, "%s_m%d", kind_name(kind), m);   // one shape per format
    else snprintf(buf, len, "%s_m%d_g%d_r%d", kind_name(kind), m, G, qg::kRowSlots);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by the call and by qg_variant_name.
qg_status check_shape(int fmt, int64_t m, int64_t N, int64_t K, qg::Layout* L)
{
    if (m < 1 || m > 4) return QG_ERR_UNSUPPORTED;
    if (!qg::make_layout(fmt, N, K, L)) return QG_ERR_INVALID_ARG;
    if (qg::lds_bytes_for(*L, int(m)) > qg::kMaxDynLdsBytes) return QG_ERR_UNSUPPORTED;
    return QG_OK;
}

// Gate/up pair layout for N gate rows (same m = 1 LDS rule as the GEMV).
qg_status check_gate_up(int64_t N, int64_t K, qg::Layout* L)
{
    int64_t rps;
    if (!qg::make_gate_up_layout(N, K, L, &rps)) return QG_ERR_INVALID_ARG;
    if (qg::lds_bytes_for(*L, 1) > qg::kMaxDynLdsBytes) return QG_ERR_UNSUPPORTED;
    return QG_OK;
}

// Dense GEMV; with idx_out the argmax epilogue (y may then be null).
// Matrix-core GEMV (MmaLayout), m = 2..16 (any K: rows of x too long to
// stage in LDS are read from memory).
qg_status check_mma(int fmt, int64_t m, int64_t N, int64_t K, qg::MmaLayout* L)
{
    // Single-token decode (m = 1) is the VALU kernels' job: the matrix cores
    // start at two rows.
    if (m < 2 || m > 16) return QG_ERR_UNSUPPORTED;
    if (!qg::make_mma_layout(fmt, N, K, L)) return QG_ERR_INVALID_ARG;
    return QG_OK;
}

qg_status run_mma(int fmt, int kind, const void* w_packed, const uint16_t* x, float* y, int64_t m,
                  int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* stream)
{
    if (!w_packed || !x || !y) return QG_ERR_INVALID_ARG;
    if (m == 0) return QG_OK;
    qg::MmaLayout L;
    const qg_status st = check_mma(fmt, m, N, K, &L);
    if (st != QG_OK) return st;
    if (ldx < K || ldy < N) return QG_ERR_INVALID_ARG;
    if (!aligned(w_packed, 256) || !aligned(x, 4) || !aligned(y, 4)) return QG_ERR_ALIGNMENT;
    if (m > 1 && (ldx % 2) != 0) return QG_ERR_ALIGNMENT;
    qg::MmaParams kp;
    kp.w = static_cast<const uint8_t*>(w_packed);
    kp.x = x;
    kp.y = y;
    kp.ldx = ldx;
    kp.ldy = ldy;
    kp.m = int32_t(m);
    kp.N = int32_t(N);
    kp.K = K;
    kp.J = L.J;
    kp.tiles = L.tiles;
    kp.code_bytes = L.code_bytes;
    kp.meta_tile_bytes = L.meta_tile_bytes;
    kp.tiles_q = kp.tiles_r = 0;   // set per launch shape
    kp.inv_cpr = 1.0f / float(K / 8);
    // LDS a work-group needs to stage x: m bf16 rows, and for Q4G32 also
    // the rows' sums over each 32-group (K / 32 groups x 16 rows of fp32).
    const size_t staged = size_t(m) * size_t(K) * 2 + (fmt == qg::FMT_Q4G32 ? size_t(K) * 2 : 0);
    (void)hipGetLastError();
    if (qg::launch_mma_sized(fmt, kp, staged, static_cast<hipStream_t>(stream)) != hipSuccess)
        return QG_ERR_HIP;
    g_route[kind][m - 1][0].fetch_add(1, std::memory_order_relaxed);
    return QG_OK;
}

// The checks of a dense call (m >= 1) that do not involve the argmax
// workspace; with idx_out the argmax epilogue (y may then be null).
qg_status validate_dense(int fmt, const void* w_packed, const uint16_t* x, const float* y,
                         const int32_t* idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                         int64_t ldy, qg::Layout* L)
{
    const bool argmax = idx_out != nullptr;
    if (!w_packed || !x || (!y && !argmax)) return QG_ERR_INVALID_ARG;
    const qg_status st = check_shape(fmt, m, N, K, L);
    if (st != QG_OK) return st;
    if (ldx < K || (y && ldy < N)) return QG_ERR_INVALID_ARG;
    if (!aligned(w_packed, 256) || !aligned(x, 4) || (y && !aligned(y, 4))) return QG_ERR_ALIGNMENT;
    if (argmax && !aligned(idx_out, 4)) return QG_ERR_ALIGNMENT;
    if (m > 1 && (ldx % 2) != 0) return QG_ERR_ALIGNMENT;
    return QG_OK;
}

qg_status run_dense(int fmt, const void* w_packed, const uint16_t* x, float* y, int64_t m,
                    int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* stream,
                    int32_t* idx_out = nullptr, void* workspace = nullptr, size_t workspace_bytes = 0)
{
    const bool argmax = idx_out != nullptr;
    if (argmax && !workspace) return QG_ERR_INVALID_ARG;
    if (m == 0 && w_packed && x && (y || argmax)) return QG_OK;  // an empty batch: nothing to compute
    qg::Layout L;
    const qg_status st = validate_dense(fmt, w_packed, x, y, idx_out, m, N, K, ldx, ldy, &L);
    if (st != QG_OK) return st;
    if (argmax && workspace_bytes < qg::argmax_workspace_bytes(m)) return QG_ERR_INVALID_ARG;
    if (argmax && !aligned(workspace, 8)) return QG_ERR_ALIGNMENT;
    qg::LaunchArgs a;
    a.layout = L;
    a.grouped = false;
    a.m = int(m);
    a.w = w_packed;
    a.expert_stride = 0;
    a.ids = nullptr;
    a.n_experts = 1;
    a.n_slots = 1;
    a.x = x;
    a.ldx = ldx;
    a.x_slot_stride = 0;
    a.y = y;
    a.ldy = ldy;
    a.y_slot_stride = 0;
    a.swiglu = false;
    a.act = nullptr;
    a.act_slot_stride = 0;
    a.n_out = N;
    a.argmax = argmax;
    a.idx_out = idx_out;
    a.argmax_workspace = workspace;
    a.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    if (qg::launch(a) != hipSuccess) return QG_ERR_HIP;
    const int kind = argmax ? (fmt == qg::FMT_Q8G64 ? 6 : 7) : kind_of(fmt);
    g_route[kind][m - 1][log2i(L.G)].fetch_add(1, std::memory_order_relaxed);
    return QG_OK;
}

// --------------------------------------------------------------------------
// Library-owned argmax scratch, for the allocation-free LM-head call
// (qgemv_q8g64_argmax_noalloc): the fused argmax's keys and finished-work-
// group counter (qg::argmax_workspace_bytes(m) <= 48 bytes for m <= 4).
// One copy per GPU, held until the process ends.  Every completed call
// leaves the bytes it used at zero (its last work-group clears them), and
// the first call on a device zeroes the whole array with a fill kernel
// before anything reads it, so every call starts from zeros.  Calls that
// overlap in time on one GPU share the array and race.
constexpr size_t kScratchBytes = 256;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void scratch_zero(unsigned char* p, size_t n)
{
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of this GPU's `scratch` (the host-side name is only a
// stand-in for it), looked up once per device with that device current; the
// first lookup also enqueues the zero fill on the caller's stream.
qg_status scratch_for_current_device(hipStream_t stream, void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QG_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return QG_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return QG_ERR_HIP;
        }
        (void)hipGetLastError();
        hipLaunchKernelGGL(scratch_zero, dim3(1), dim3(256), 0, stream,
                           static_cast<unsigned char*>(ptr), kScratchBytes);
        if (hipGetLastError() != hipSuccess) return QG_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QG_OK;
}

}  // namespace

extern "C" {

const char* qg_status_string(qg_status status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_ERR_INVALID_ARG: return "invalid argument";
    case QG_ERR_UNSUPPORTED: return "unsupported";
    case QG_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case QG_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int qg_abi_version(void) { return QG_ABI_VERSION; }

qg_status qgemv_q8g64(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                      int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_dense(qg::FMT_Q8G64, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q4g32(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                      int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_dense(qg::FMT_Q4G32, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q8g128(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                       int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_dense(qg::FMT_Q8G128, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q8pc(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                     int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_dense(qg::FMT_Q8PC, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_grouped_q4g32(const void* w_experts_packed, int64_t expert_stride_bytes,
                              int32_t n_experts, const int32_t* expert_ids_dev, int32_t n_slots,
                              const uint16_t* x_bf16, int64_t x_slot_stride, float* y,
                              int64_t y_slot_stride, int64_t N, int64_t K, void* hip_stream)
{
    if (!w_experts_packed || !expert_ids_dev || !x_bf16 || !y) return QG_ERR_INVALID_ARG;
    if (n_slots == 0) return QG_OK;  // no routed experts: nothing to compute
    if (n_slots < 0 || n_slots > 64) return QG_ERR_UNSUPPORTED;
    if (n_experts < 1) return QG_ERR_INVALID_ARG;
    qg::Layout L;
    const qg_status st = check_shape(qg::FMT_Q4G32, 1, N, K, &L);
    if (st != QG_OK) return st;
    if (expert_stride_bytes < L.total_bytes || x_slot_stride < 0 || y_slot_stride < N)
        return QG_ERR_INVALID_ARG;
    if (expert_stride_bytes % 256 != 0 || x_slot_stride % 2 != 0) return QG_ERR_ALIGNMENT;
    if (!aligned(w_experts_packed, 256) || !aligned(x_bf16, 4) || !aligned(y, 4) ||
        !aligned(expert_ids_dev, 4))
        return QG_ERR_ALIGNMENT;
    qg::LaunchArgs a;
    a.layout = L;
    a.grouped = true;
    a.m = 1;
    a.w = w_experts_packed;
    a.expert_stride = expert_stride_bytes;
    a.ids = expert_ids_dev;
    a.n_experts = n_experts;
    a.n_slots = n_slots;
    a.x = x_bf16;
    a.ldx = K;
    a.x_slot_stride = x_slot_stride;
    a.y = y;
    a.ldy = N;
    a.y_slot_stride = y_slot_stride;
    a.swiglu = false;
    a.act = nullptr;
    a.act_slot_stride = 0;
    a.n_out = N;
    a.argmax = false;
    a.idx_out = nullptr;
    a.argmax_workspace = nullptr;
    a.stream = static_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    if (qg::launch(a) != hipSuccess) return QG_ERR_HIP;
    g_route[2][0][log2i(L.G)].fetch_add(1, std::memory_order_relaxed);
    return QG_OK;
}

qg_status qgemv_grouped_q4g32_swiglu(const void* w_gate_up_packed, int64_t expert_stride_bytes,
                                     int32_t n_experts, const int32_t* expert_ids_dev,
                                     int32_t n_slots, const uint16_t* x_bf16,
                                     int64_t x_slot_stride, uint16_t* act_bf16,
                                     int64_t act_slot_stride, int64_t N, int64_t K,
                                     void* hip_stream)
{
    if (!w_gate_up_packed || !expert_ids_dev || !x_bf16 || !act_bf16) return QG_ERR_INVALID_ARG;
    if (n_slots == 0) return QG_OK;
    if (n_slots < 0 || n_slots > 64) return QG_ERR_UNSUPPORTED;
    if (n_experts < 1) return QG_ERR_INVALID_ARG;
    qg::Layout L;
    const qg_status st = check_gate_up(N, K, &L);
    if (st != QG_OK) return st;
    if (expert_stride_bytes < L.total_bytes || x_slot_stride < 0 || act_slot_stride < N)
        return QG_ERR_INVALID_ARG;
    if (expert_stride_bytes % 256 != 0 || x_slot_stride % 2 != 0) return QG_ERR_ALIGNMENT;
    if (!aligned(w_gate_up_packed, 256) || !aligned(x_bf16, 4) || !aligned(act_bf16, 2) ||
        !aligned(expert_ids_dev, 4))
        return QG_ERR_ALIGNMENT;
    qg::LaunchArgs a;
    a.layout = L;
    a.grouped = true;
    a.m = 1;
    a.w = w_gate_up_packed;
    a.expert_stride = expert_stride_bytes;
    a.ids = expert_ids_dev;
    a.n_experts = n_experts;
    a.n_slots = n_slots;
    a.x = x_bf16;
    a.ldx = K;
    a.x_slot_stride = x_slot_stride;
    a.y = nullptr;
    a.ldy = L.N;
    a.y_slot_stride = 0;
    a.swiglu = true;
    a.act = act_bf16;
    a.act_slot_stride = act_slot_stride;
    a.n_out = N;
    a.argmax = false;
    a.idx_out = nullptr;
    a.argmax_workspace = nullptr;
    a.stream = static_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    if (qg::launch(a) != hipSuccess) return QG_ERR_HIP;
    g_route[5][0][log2i(L.G)].fetch_add(1, std::memory_order_relaxed);
    return QG_OK;
}

qg_status qgemv_q8g64_argmax(const void* w_packed, const uint16_t* x_bf16, float* logits,
                             int32_t* idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                             int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (!idx_out) return QG_ERR_INVALID_ARG;
    return run_dense(qg::FMT_Q8G64, w_packed, x_bf16, logits, m, N, K, ldx, ldy, hip_stream, idx_out,
                     workspace, workspace_bytes);
}

qg_status qgemv_q8g128_argmax(const void* w_packed, const uint16_t* x_bf16, float* logits,
                              int32_t* idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                              int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (!idx_out) return QG_ERR_INVALID_ARG;
    return run_dense(qg::FMT_Q8G128, w_packed, x_bf16, logits, m, N, K, ldx, ldy, hip_stream,
                     idx_out, workspace, workspace_bytes);
}

qg_status qgemv_q8g64_argmax_noalloc(const void* w_packed, const uint16_t* x_bf16, float* logits,
                                     int32_t* idx_out, int64_t m, int64_t N, int64_t K, int64_t ldx,
                                     int64_t ldy, void* hip_stream)
{
    // Everything the call itself would reject is rejected first, before the
    // scratch is touched; the scratch holds the workspace of up to 4 rows.
    if (!idx_out || !w_packed || !x_bf16) return QG_ERR_INVALID_ARG;
    if (m == 0) return QG_OK;
    if (m < 1 || m > 4 || qg::argmax_workspace_bytes(m) > kScratchBytes) return QG_ERR_UNSUPPORTED;
    qg::Layout L;
    const qg_status st = validate_dense(qg::FMT_Q8G64, w_packed, x_bf16, logits, idx_out, m, N, K, ldx,
                                        ldy, &L);
    if (st != QG_OK) return st;
    void* ws = nullptr;
    const qg_status sst = scratch_for_current_device(static_cast<hipStream_t>(hip_stream), &ws);
    if (sst != QG_OK) return sst;
    return run_dense(qg::FMT_Q8G64, w_packed, x_bf16, logits, m, N, K, ldx, ldy, hip_stream, idx_out, ws,
                     kScratchBytes);
}

qg_status qgemv_q8g64_mma(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                          int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_mma(qg::FMT_Q8G64, 8, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q8g128_mma(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                           int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_mma(qg::FMT_Q8G128, 9, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q4g32_mma(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                          int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_mma(qg::FMT_Q4G32, 11, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

qg_status qgemv_q8pc_mma(const void* w_packed, const uint16_t* x_bf16, float* y, int64_t m,
                         int64_t N, int64_t K, int64_t ldx, int64_t ldy, void* hip_stream)
{
    return run_mma(qg::FMT_Q8PC, 10, w_packed, x_bf16, y, m, N, K, ldx, ldy, hip_stream);
}

size_t qg_argmax_workspace_size(int64_t m)
{
    if (m < 0 || m > 65535) return 0;
    return qg::argmax_workspace_bytes(m);
}

qg_status qg_argmax_f32(const float* x, int64_t m, int64_t N, int64_t ldx, int32_t* idx_out,
                        void* workspace, size_t workspace_bytes, void* hip_stream)
{
    if (!x || !idx_out || !workspace) return QG_ERR_INVALID_ARG;
    if (m == 0) return QG_OK;
    if (m < 0 || m > 65535 || N < 1 || N > (int64_t(1) << 31) - 1 || ldx < N)
        return QG_ERR_INVALID_ARG;
    if (workspace_bytes < qg::argmax_workspace_bytes(m)) return QG_ERR_INVALID_ARG;
    if (!aligned(x, 4) || !aligned(idx_out, 4) || !aligned(workspace, 8)) return QG_ERR_ALIGNMENT;
    (void)hipGetLastError();
    if (qg::launch_argmax(x, m, N, ldx, idx_out, workspace, static_cast<hipStream_t>(hip_stream)) !=
        hipSuccess)
        return QG_ERR_HIP;
    return QG_OK;
}

void qg_route_counts_reset(void)
{
    for (int k = 0; k < kKinds; ++k)
        for (int m = 0; m < kMs; ++m)
            for (int g = 0; g < kGs; ++g) g_route[k][m][g].store(0);
}

uint64_t qg_route_count(const char* variant)
{
    if (!variant) return 0;
    char buf[64];
    for (int k = 0; k < kKinds; ++k)
        for (int m = 0; m < kMs; ++m)
            for (int g = 0; g < kGs; ++g) {
                format_variant(k, m + 1, 1 << g, buf, sizeof buf);
                if (strcmp(buf, variant) == 0) return g_route[k][m][g].load();
            }
    return 0;
}

qg_status qg_read_stream(const void* buf, size_t bytes, uint32_t* sink, int32_t waves_per_cu,
                         void* hip_stream)
{
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || waves_per_cu < 0 || waves_per_cu > 32)
        return QG_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return QG_ERR_ALIGNMENT;
    (void)hipGetLastError();
    if (qg::launch_read_stream(buf, int64_t(bytes / 16), sink, waves_per_cu ? waves_per_cu : 8,
                               static_cast<hipStream_t>(hip_stream)) != hipSuccess)
        return QG_ERR_HIP;
    return QG_OK;
}

qg_status qg_set_launch_override(int64_t target_waves, int32_t contig, int32_t ring_depth)
{
    if (target_waves < 0 || target_waves > (int64_t(1) << 24) || contig < -1 || contig > 1 ||
        (ring_depth != 0 && ring_depth != 1 && ring_depth != 2 && ring_depth != 4))
        return QG_ERR_INVALID_ARG;
    qg::LaunchOverride o;
    o.use_policy = 1;
    o.target_waves = target_waves;
    o.contig = contig;
    o.shape = ring_depth == 2   ? qg::SHAPE_D2_W4
              : ring_depth == 4 ? qg::SHAPE_D4_W4
              : ring_depth == 1 ? qg::SHAPE_XR
                                : -1;
    qg::set_launch_override(o);
    return QG_OK;
}

qg_status qg_set_wave_trace(void* device_records, int64_t capacity_records)
{
    if (device_records && (capacity_records <= 0 || reinterpret_cast<uintptr_t>(device_records) % 8 != 0))
        return QG_ERR_INVALID_ARG;
    qg::set_wave_trace(device_records, capacity_records);
    return QG_OK;
}

qg_status qg_wave_trace_state(int64_t* records, int64_t* launches, int64_t* dropped)
{
    if (!records || !launches || !dropped) return QG_ERR_INVALID_ARG;
    qg::wave_trace_state(records, launches, dropped);
    return QG_OK;
}

qg_status qg_variant_name(int fmt, int64_t m, int64_t N, int64_t K, char* buf, size_t buf_len)
{
    if (!buf || buf_len == 0) return QG_ERR_INVALID_ARG;
    static const int kind_format[kKinds] = {qg::FMT_Q8G64, qg::FMT_Q4G32, qg::FMT_Q4G32,
                                            qg::FMT_Q8G128, qg::FMT_Q8PC, qg::FMT_Q4G32,
                                            qg::FMT_Q8G64, qg::FMT_Q8G128, qg::FMT_Q8G64,
                                            qg::FMT_Q8G128, qg::FMT_Q8PC, qg::FMT_Q4G32};
    if (fmt < 0 || fmt >= kKinds) return QG_ERR_INVALID_ARG;
    if (fmt >= 8) {
        qg::MmaLayout ML;
        const qg_status sm = check_mma(kind_format[fmt], m, N, K, &ML);
        if (sm != QG_OK) return sm;
        format_variant(fmt, int(m), 4, buf, buf_len);
        return QG_OK;
    }
    if ((fmt == 2 || fmt == 5) && m != 1) return QG_ERR_UNSUPPORTED;
    qg::Layout L;
    const qg_status st = fmt == 5 ? check_gate_up(N, K, &L) : check_shape(kind_format[fmt], m, N, K, &L);
    if (st != QG_OK) return st;
    format_variant(fmt, int(m), L.G, buf, buf_len);
    return QG_OK;
}

}  // extern "C"
