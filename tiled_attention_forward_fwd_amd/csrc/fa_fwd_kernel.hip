// fa_fwd_kernel.hip -- host dispatch of the attention forward without masks:
// workgroup shape, direct and split launches (kernels in fa_fwd_kernel.h).

#include "fa_fwd_kernel.h"

namespace fa {

// Workgroup shape per problem. 256-row workgroups (8 waves) stream each K/V
// tile from L2 once for twice the rows, which lowers L2 and LDS-fill traffic
// and, the chip being power-limited under this load, raises the clock it
// holds; they are used for non-causal problems whose grid still gives every
// CU a workgroup. Causal problems keep 128-row workgroups (less work above
// the diagonal), as do small grids.
Shape pick_shape(int B, int H, int n_queries, int d, bool causal)
{
    (void)d;
    Shape sh;
    sh.waves = 4;
    sh.rows_per_wave = 32;
    if (!causal) {
        const int64_t wg256 = (int64_t)B * H * ((n_queries + 255) / 256);
        if (wg256 >= 256) sh.waves = 8;
    }
    sh.block_m = sh.waves * sh.rows_per_wave;
    sh.threads = 64 * sh.waves;
    return sh;
}

int block_n(int) { return 64; }
int lds_bytes(int d) { return 4 * 64 * d * 2; }

hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int H, int Nq, int Nk, int d, bool causal, float scale, bool bf16,
                            int n_splits, float* workspace, hipStream_t stream)
{
    const int BH = B * H;
#define FA_DISPATCH(T, D)                                                                         \
    return causal ? launch_split<T, D, true, false>(q, k, v, o, lse, BH, Nq, Nk, scale, n_splits,  \
                                                    workspace, MaskArgs{}, stream)                 \
                  : launch_split<T, D, false, false>(q, k, v, o, lse, BH, Nq, Nk, scale, n_splits, \
                                                     workspace, MaskArgs{}, stream)
    if (bf16) {
        if (d == 64) FA_DISPATCH(__bf16, 64);
        FA_DISPATCH(__bf16, 128);
    }
    if (d == 64) FA_DISPATCH(_Float16, 64);
    FA_DISPATCH(_Float16, 128);
#undef FA_DISPATCH
}

int split_rows_per_tile() { return 128; }

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, bool causal, float scale, bool bf16,
                      hipStream_t stream)
{
    const int BH = B * H;
    const Shape sh = pick_shape(B, H, Nq, d, causal);
#define FA_DISPATCH(T, D)                                                                        \
    return causal ? launch_shape<T, D, true, false>(sh, q, k, v, o, lse, BH, Nq, Nk, scale,      \
                                                    MaskArgs{}, stream)                           \
                  : launch_shape<T, D, false, false>(sh, q, k, v, o, lse, BH, Nq, Nk, scale,     \
                                                     MaskArgs{}, stream)
    if (bf16) {
        if (d == 64) FA_DISPATCH(__bf16, 64);
        FA_DISPATCH(__bf16, 128);
    }
    if (d == 64) FA_DISPATCH(_Float16, 64);
    FA_DISPATCH(_Float16, 128);
#undef FA_DISPATCH
}

}  // namespace fa
