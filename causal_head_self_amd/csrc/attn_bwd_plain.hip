// attn_bwd_plain.hip -- the one-launch backward at head dim 64 without dropout
// (attn_bwd_d64_kernel<false, false, false> of attn_bf16_d64.hip), instantiated in a
// translation unit of its own so that the build can compile it with another
// instruction-scheduling strategy than the other kernels: LLVM's iterative ILP
// scheduler, which interleaves this kernel's MFMA and VALU work more closely
// (backward 64.7 -> 62.7 us at B8 H12 T1024 D64 bf16, no spills).  The other
// kernels keep the default scheduler: under the ILP one the forward is slower and
// the dropout and head-dim-128 backward kernels spill hundreds of VGPRs.
#define CATTN_D64_KERNELS_ONLY
#include "attn_bf16_d64.hip"

namespace cattn {
namespace d64 {
template __global__ void attn_bwd_d64_kernel<false, false, false>(BwdParams, int, int, NoRope);
}  // namespace d64
}  // namespace cattn
