// LM-head GEMV with the greedy argmax fused into its epilogue: the
// instantiations of kernel_body.h for the two LM-head formats (own
// translation unit so it compiles in parallel with the plain formats).
#include "kernel_body.h"

namespace qg {

hipError_t launch_argmax_epilogue(int fmt, int m, int G, int shape, const KernelParams& kp,
                                  int64_t waves, size_t lds, hipStream_t s)
{
    switch (fmt) {
    case FMT_Q8G64: return launch_argmax_format<FMT_Q8G64>(m, G, shape, kp, waves, lds, s);
    case FMT_Q8G128: return launch_argmax_format<FMT_Q8G128>(m, G, shape, kp, waves, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qg
