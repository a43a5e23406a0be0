// The greedy-choice key shared by the argmax kernels: one unsigned 64-bit
// number whose order is the (value, lower index) order of fp32 logits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// High 32 bits: the value's total order (-inf lowest, -0 folded onto +0,
// every NaN above +inf).  Low 32 bits: the inverted index, so that among
// equal values the lower index has the larger key.  No value maps to key 0,
// which therefore starts every reduction.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx)
{
    uint32_t u = __float_as_uint(v);
    uint32_t ord;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        ord = 0xffffffffu;
    } else {
        if (u == 0x80000000u) u = 0;
        ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return (uint64_t(ord) << 32) | uint64_t(~idx);
}

__device__ __forceinline__ uint64_t max_key(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Index held by a key.
__device__ __forceinline__ int32_t key_index(uint64_t k) { return int32_t(~uint32_t(k & 0xffffffffu)); }

}  // namespace qg
