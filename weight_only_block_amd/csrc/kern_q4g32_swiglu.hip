// Grouped Q4G32 gate/up kernels with the SwiGLU epilogue: the
// instantiations of kernel_body.h for that call (own translation unit so it
// compiles in parallel with the plain formats).
#include "kernel_body.h"

namespace qg {

hipError_t launch_q4g32_swiglu(int G, int shape, const KernelParams& kp, int64_t waves, int slots,
                               size_t lds, hipStream_t s)
{
    return launch_swiglu<FMT_Q4G32>(G, shape, kp, waves, slots, lds, s);
}

}  // namespace qg
