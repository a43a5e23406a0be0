// Internal interface between the C ABI (abi.cpp) and the kernels
// (kernels.hip).  Not installed; callers use include/qgemv.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace qg {

// LDS a work-group may use on gfx950.
constexpr size_t kMaxLdsBytes = 160 * 1024;

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
    int64_t code_bytes;        // offset of the meta blocks
    int64_t meta_step_bytes;
    int64_t contig_k;          // > 0: each wave streams contig_k consecutive tiles
};

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
    hipStream_t stream;
};

// Bytes of dynamic LDS a launch of this layout needs for m activation rows.
size_t lds_bytes_for(const Layout& L, int m);

// Enqueues the kernel; returns the HIP status of the launch.
hipError_t launch(const LaunchArgs& a);

}  // namespace qg
