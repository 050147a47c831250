// fa_fwd_masked.hip -- the attention forward with padding lengths and sliding
// windows at head dims 64 and 128 (fa_fwd_kernel.h with MASKS = true), direct
// and split-key launches. The workgroup shape and the split layout are those
// of the unmasked launches, except that a kernel head dim of 128 keeps 4 waves.

#include "fa_fwd_kernel.h"

namespace fa {

// The 8-wave d=128 kernel already holds 256 VGPRs without masks; the per-row
// key ranges would make it spill, so masked d=128 keeps 128-row workgroups.
Shape pick_shape_masked(int B, int H, int n_queries, int d, bool causal)
{
    Shape sh = pick_shape(B, H, n_queries, d, causal);
    if (kernel_dim(d) == 128 && sh.waves == 8) {
        sh.waves = 4;
        sh.block_m = sh.waves * sh.rows_per_wave;
        sh.threads = 64 * sh.waves;
    }
    return sh;
}

hipError_t launch_forward_masked(const FwdArgs& a) { return launch_variant<true, false>(a); }

}  // namespace fa
