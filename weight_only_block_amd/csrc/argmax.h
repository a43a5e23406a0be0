// Internal interface of the greedy argmax kernel (argmax.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qg {

// Workspace bytes for m rows: m 64-bit keys, then m 32-bit counters.
size_t argmax_workspace_bytes(int64_t m);

// Enqueues the argmax of m rows of N fp32 values (row stride ldx) into
// out[m]; workspace holds argmax_workspace_bytes(m) zero bytes and is left
// zeroed when the kernel completes.
hipError_t launch_argmax(const float* x, int64_t m, int64_t N, int64_t ldx, int32_t* out,
                         void* workspace, hipStream_t s);

}  // namespace qg
