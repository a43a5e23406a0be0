// Internal interface of the plain read stream (read_stream.hip), the
// bandwidth reference exported as qg_read_stream.  Not installed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// A lane whose XOR fold of the units it read equals this writes it to the sink.
constexpr uint32_t kReadStreamPattern = 0x9E3779B9u;

// Reads `units` 16-byte units at buf with waves_per_cu waves per compute
// unit of the current device.
hipError_t launch_read_stream(const void* buf, int64_t units, uint32_t* sink, int waves_per_cu,
                              hipStream_t s);

}  // namespace qg
