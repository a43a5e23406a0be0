// Q4G32 kernels: the instantiations of kernel_body.h for this format
// (one translation unit per format so they compile in parallel).
#include "kernel_body.h"

namespace qg {

hipError_t launch_q4g32(int m, bool grouped, int G, int shape, const KernelParams& kp, int64_t waves,
                       int slots, size_t lds, hipStream_t s)
{
    return launch_format<FMT_Q4G32>(m, grouped, G, shape, kp, waves, slots, lds, s);
}

}  // namespace qg
