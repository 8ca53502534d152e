// The unmasked bf16 ping-pong attention kernel (grids of whole blocks, no token window), the
// instantiation every divisible grid runs. It sits in a translation unit of its own because it is
// compiled with LLVM's iterative ILP machine scheduler (-amdgpu-sched-strategy=iterative-ilp), which
// interleaves its LDS operand reads with the MFMAs better than the default scheduler; the masked
// variants keep the default, under which they spill fewer registers.
#include "attn_fwd_impl.h"

namespace lcsa {

void launch_attn_fwd_pp_dense(const AttnArgs& a, int head_dim, hipStream_t s) {
  if (head_dim == 128)
    attn_fwd_pp_kernel<128, kMaskNone><<<a.nwg, 512, 0, s>>>(a);
  else
    attn_fwd_pp_kernel<64, kMaskNone><<<a.nwg, 512, 0, s>>>(a);
}

}  // namespace lcsa
