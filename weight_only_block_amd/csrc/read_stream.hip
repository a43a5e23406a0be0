// Plain HBM read stream: the reference a weight-streaming kernel is compared
// with (its bandwidth on the same part, same access width).  Not part of
// the GEMV path; the library exports it as a measurement hook.
//
// Every lane reads 16-byte units with non-temporal loads.  A wave takes
// chunks of 8 KiB (512 units): lane l reads units l, l + 64, ..., l + 448
// of the chunk, so each of its eight loads in flight is one contiguous KiB
// across the wave, and consecutive loads continue where the last ended, as
// a GEMV wave streams the items of a tile.  Waves take chunks grid-stride,
// so at any moment the launch reads one window of the buffer.  The units
// are XOR-folded per lane; a lane whose fold equals a fixed pattern stores
// it to the sink, which keeps every load live (and lets a test check that
// the data was read).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "read_stream.h"

namespace qg {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadWaves = 4;                 // waves per work-group
constexpr int kChunkLoads = 8;                // loads per lane per chunk
constexpr int64_t kChunkUnits = 64 * kChunkLoads;

__global__ __launch_bounds__(64 * kReadWaves) void read_stream_kernel(const u32x4* __restrict__ p, int64_t n,
                                                                      uint32_t* sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = int64_t(blockIdx.x) * kReadWaves + (threadIdx.x >> 6);
    const int64_t waves = int64_t(gridDim.x) * kReadWaves;
    const int64_t full = n / kChunkUnits;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = wave; c < full; c += waves) {
        const u32x4* q = p + c * kChunkUnits + lane;
        u32x4 v[kChunkLoads];
#pragma unroll
        for (int u = 0; u < kChunkLoads; ++u) v[u] = __builtin_nontemporal_load(q + 64 * u);
#pragma unroll
        for (int u = 0; u < kChunkLoads; ++u) acc ^= v[u];
    }
    // The partial chunk at the end (fewer than 512 units) goes to the wave
    // next in line after the full chunks.
    if (wave == full % waves) {
        for (int64_t i = full * kChunkUnits + lane; i < n; i += 64) acc ^= __builtin_nontemporal_load(p + i);
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == kReadStreamPattern) *sink = r;
}

int64_t device_compute_units()
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

}  // namespace

hipError_t launch_read_stream(const void* buf, int64_t units, uint32_t* sink, int waves_per_cu, hipStream_t s)
{
    const int64_t waves = device_compute_units() * waves_per_cu;
    const int64_t chunks = (units + kChunkUnits - 1) / kChunkUnits;
    int64_t blocks = (waves + kReadWaves - 1) / kReadWaves;
    const int64_t need = (chunks + kReadWaves - 1) / kReadWaves;
    if (blocks > need) blocks = need;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(blocks)), dim3(64 * kReadWaves), 0, s,
                       static_cast<const u32x4*>(buf), units, sink);
    return hipGetLastError();
}

}  // namespace qg
