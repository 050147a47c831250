// fa_bwd_hdim.hip -- the backward pass at head dims below 128 other than 64
// (a multiple of 8), run PADDED with the d = 64 or d = 128 kernels of
// fa_bwd_kernel.h.
#include "fa_bwd_kernel.h"

namespace fa {

hipError_t launch_bwd_hdim(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H, int Nq,
                           int Nk, int d, bool causal, float scale, bool bf16, const MaskArgs* mask,
                           hipStream_t stream)
{
    return launch_bwd_variant<true>(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d, causal, scale,
                                    bf16, mask, stream);
}

}  // namespace fa
