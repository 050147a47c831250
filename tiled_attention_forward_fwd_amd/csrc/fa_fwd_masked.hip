// fa_fwd_masked.hip -- host dispatch of the attention forward with padding
// lengths and sliding windows (kernels in fa_fwd_kernel.h, MASKS = true). The
// workgroup shape and the split layout are those of the unmasked launches.

#include "fa_fwd_kernel.h"

namespace fa {

// The 8-wave d=128 kernel already holds 256 VGPRs without masks; the per-row
// key ranges would make it spill, so masked d=128 keeps 128-row workgroups.
Shape pick_shape_masked(int B, int H, int n_queries, int d, bool causal)
{
    Shape sh = pick_shape(B, H, n_queries, d, causal);
    if (d == 128 && sh.waves == 8) {
        sh.waves = 4;
        sh.block_m = sh.waves * sh.rows_per_wave;
        sh.threads = 64 * sh.waves;
    }
    return sh;
}

hipError_t launch_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                             int H, int Nq, int Nk, int d, bool causal, const MaskArgs& mask,
                             float scale, bool bf16, hipStream_t stream)
{
    const int BH = B * H;
    const Shape sh = pick_shape_masked(B, H, Nq, d, causal);
#define FA_DISPATCH(T, D)                                                                          \
    return causal ? launch_shape<T, D, true, true>(sh, q, k, v, o, lse, BH, Nq, Nk, scale, mask,   \
                                                   stream)                                         \
                  : launch_shape<T, D, false, true>(sh, q, k, v, o, lse, BH, Nq, Nk, scale, mask,  \
                                                    stream)
    if (bf16) {
        if (d == 64) FA_DISPATCH(__bf16, 64);
        FA_DISPATCH(__bf16, 128);
    }
    if (d == 64) FA_DISPATCH(_Float16, 64);
    FA_DISPATCH(_Float16, 128);
#undef FA_DISPATCH
}

hipError_t launch_fwd_split_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int d, bool causal,
                                   const MaskArgs& mask, float scale, bool bf16, int n_splits,
                                   float* workspace, hipStream_t stream)
{
    const int BH = B * H;
#define FA_DISPATCH(T, D)                                                                          \
    return causal ? launch_split<T, D, true, true>(q, k, v, o, lse, BH, Nq, Nk, scale, n_splits,   \
                                                   workspace, mask, stream)                        \
                  : launch_split<T, D, false, true>(q, k, v, o, lse, BH, Nq, Nk, scale, n_splits,  \
                                                    workspace, mask, stream)
    if (bf16) {
        if (d == 64) FA_DISPATCH(__bf16, 64);
        FA_DISPATCH(__bf16, 128);
    }
    if (d == 64) FA_DISPATCH(_Float16, 64);
    FA_DISPATCH(_Float16, 128);
#undef FA_DISPATCH
}

}  // namespace fa
