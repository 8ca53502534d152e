// The bf16 attention kernel for block-granular masks: whole blocks (kMaskNone, every grid
// that is a multiple of 8, with or without a block window) and partial edge blocks (kMaskRagged).
// These instantiations sit in a translation unit of their own because they are compiled with LLVM's
// iterative ILP machine scheduler (-amdgpu-sched-strategy=iterative-ilp), which spreads their LDS
// operand reads between the MFMAs better than the default scheduler (7% faster on both); the
// token-window variant keeps the default, under which it spills fewer registers.
#include "attn_fwd_impl.h"

namespace lcsa {

void launch_attn_fwd_bf16_block(const AttnArgs& a, int head_dim, bool ragged, hipStream_t s) {
  if (head_dim == 128) {
    if (ragged) attn_fwd_bf16_kernel<128, kMaskRagged><<<a.nwg, 256, 0, s>>>(a);
    else attn_fwd_bf16_kernel<128, kMaskNone><<<a.nwg, 256, 0, s>>>(a);
  } else {
    if (ragged) attn_fwd_bf16_kernel<64, kMaskRagged><<<a.nwg, 256, 0, s>>>(a);
    else attn_fwd_bf16_kernel<64, kMaskNone><<<a.nwg, 256, 0, s>>>(a);
  }
}

}  // namespace lcsa
