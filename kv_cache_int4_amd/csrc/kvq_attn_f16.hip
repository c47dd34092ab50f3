// The fp16-cache comparator of the decode-step attention: its split kernel
// in a translation unit of its own, so that it keeps the compiler's default
// register assignment for matrix results (the int4 kernels' source is built
// with matrix results in VGPRs, which helps them and not this one).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_attn_kernels.hpp"

namespace kvq {

hipError_t launch_attn_split_f16(const AttnArgs& a, int nh, unsigned nsplit, hipStream_t stream) {
  if (nh == 2) hipLaunchKernelGGL((attn_split_kernel<false, KVQ_ROT_ID, 0, 2>), dim3(nsplit), dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((attn_split_kernel<false, KVQ_ROT_ID, 0, 1>), dim3(nsplit), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
