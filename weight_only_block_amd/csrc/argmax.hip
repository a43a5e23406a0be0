// Greedy token choice over fp32 logits for gfx950: per row, the index of the
// largest value, the lowest index on ties.  Each row is split across work-
// groups, as in the split argmax of the commit log of vllm.cpp pull request
// #1936, and the pieces meet through one 64-bit atomic max: a value and its
// index are packed into a key whose unsigned order is the (value, lower
// index) order, so the result does not depend on which work-group finishes
// first.  The last work-group of a row (counted with an atomic) reads the
// winner, writes the index and puts the row's workspace back to zero, so a
// call needs no separate reduce launch and no clearing launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "argmax.h"
#include "argmax_key.h"

namespace qg {

namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;                        // elements per thread per work-group
constexpr int64_t kChunk = int64_t(kThreads) * kPerThread;

__global__ __launch_bounds__(kThreads) void argmax_rows(const float* __restrict__ x, int64_t ldx,
                                                         int64_t N, int32_t* __restrict__ out,
                                                         unsigned long long* keys, unsigned int* counts)
{
    const int64_t row = blockIdx.y;
    const int64_t start = int64_t(blockIdx.x) * kChunk;
    const float* xr = x + row * ldx;
    uint64_t best = 0;
    // All loads of the chunk are issued before any compare.
    float v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t n = start + k * kThreads + threadIdx.x;
        v[k] = n < N ? xr[n] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int64_t n = start + k * kThreads + threadIdx.x;
        if (n < N) best = max_key(best, argmax_key(v[k], uint32_t(n)));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor((unsigned long long)best, off, 64);
        best = max_key(best, o);
    }
    __shared__ uint64_t wave_best[kThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_best[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) best = max_key(best, wave_best[w]);
        atomicMax(&keys[row], (unsigned long long)best);
        // The max is performed before this work-group counts itself; keys
        // are read back only through atomics, so waiting for the atomic
        // (no fence, which would write back and invalidate the whole L2)
        // is all the ordering needed.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const unsigned int done = atomicAdd(&counts[row], 1u);
        if (done == gridDim.x - 1) {
            // Every other work-group of the row has added its key: read the
            // winner and leave the workspace zeroed for the next call.
            const unsigned long long fin = atomicExch(&keys[row], 0ull);
            atomicExch(&counts[row], 0u);
            out[row] = key_index(fin);
        }
    }
}

}  // namespace

size_t argmax_workspace_bytes(int64_t m)
{
    return size_t((12 * m + 255) / 256 * 256);
}

hipError_t launch_argmax(const float* x, int64_t m, int64_t N, int64_t ldx, int32_t* out,
                         void* workspace, hipStream_t s)
{
    auto* keys = static_cast<unsigned long long*>(workspace);
    auto* counts = reinterpret_cast<unsigned int*>(keys + m);
    const dim3 grid(unsigned((N + kChunk - 1) / kChunk), unsigned(m));
    hipLaunchKernelGGL(argmax_rows, grid, dim3(kThreads), 0, s, x, ldx, N, out, keys, counts);
    return hipGetLastError();
}

}  // namespace qg
