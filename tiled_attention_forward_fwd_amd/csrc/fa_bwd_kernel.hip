// fa_bwd_kernel.hip -- the backward pass at head dims 64 and 128 (the kernels
// are in fa_bwd_kernel.h); other head dims go to fa_bwd_hdim.hip.
#include "fa_bwd_kernel.h"

namespace fa {

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq,
                      int Nk, int d, bool causal, float scale, bool bf16, const MaskArgs* mask,
                      hipStream_t stream)
{
    if (d != kernel_dim(d))
        return launch_bwd_hdim(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale, bf16,
                               mask, stream);
    return launch_bwd_variant<false>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale,
                                     bf16, mask, stream);
}

}  // namespace fa
