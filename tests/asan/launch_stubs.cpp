// launch_stubs.cpp -- host stand-ins for the three kernel launchers, so that
// the C ABI layer (argument checks, workspace layout, plan) links and runs
// under the host sanitizers without the kernel sources.  A call that passes
// every check reaches one of these and comes back as VC_ERR_DEVICE.
#include <hip/hip_runtime.h>

#include "vc_kernels.hpp"

namespace vc {

hipError_t launch_prepare_v(const TensorArg&, int, int, int, const vc_v_opts&, const WsPtrs&, hipStream_t) {
  return hipErrorUnknown;
}

hipError_t launch_prepare_qk(const TensorArg&, const TensorArg&, int, int, int, int, const WsPtrs&, hipStream_t) {
  return hipErrorUnknown;
}

hipError_t launch_attention(const AttnArgs&, const AttnTail&, hipStream_t) { return hipErrorUnknown; }

}  // namespace vc
