// fa_fwd_kernel.hip -- host side of the attention forward: workgroup shape,
// the choice among the launch variants (masks, other head dims, the key-split
// kernel for small grids), and the variant without masks at head dims 64 and
// 128 (kernels in fa_fwd_kernel.h).

#include "fa_fwd_kernel.h"

namespace fa {

// Workgroup shape per problem. 256-row workgroups (8 waves) stream each K/V
// tile from L2 once for twice the rows, which lowers L2 and LDS-fill traffic
// and, the chip being power-limited under this load, raises the clock it
// holds; they are used for non-causal problems whose grid still gives every
// CU a workgroup. Causal problems keep 128-row workgroups (less work above
// the diagonal), as do small grids and problems of at most 128 query rows: a
// 256-row workgroup would leave at least half its waves without rows while
// holding a whole CU's waves (one workgroup per CU instead of two, so half
// the K/V copies in flight; decode-like shapes, measured 25-40% slower).
Shape pick_shape(int B, int H, int n_queries, int d, bool causal)
{
    (void)d;
    Shape sh;
    sh.waves = 4;
    sh.rows_per_wave = 32;
    if (!causal && n_queries > 128) {
        const int64_t wg256 = (int64_t)B * H * ((n_queries + 255) / 256);
        if (wg256 >= 256) sh.waves = 8;
    }
    sh.block_m = sh.waves * sh.rows_per_wave;
    sh.threads = 64 * sh.waves;
    return sh;
}

int block_n(int) { return 64; }
int lds_bytes(int d, int waves, bool stage_out, bool q_tile)
{
    // two K and two V tiles (plus the Q tile of the 8-wave launches without
    // masks, padding or split); the launches without split (and head dim at
    // least 64) stage each wave's 32 output rows (D + 8 elements apart)
    // through the same memory
    const int D = kernel_dim(d);
    const int tiles = 4 * 64 * D * 2 + (q_tile ? 256 * D * 2 : 0);
    const int stage = waves * 32 * (D + 8) * 2;
    return stage_out && stage > tiles ? stage : tiles;
}
int split_rows_per_tile() { return 128; }

hipError_t launch_forward(const FwdArgs& a)
{
    const bool padded = a.d != 64 && a.d != 128;
    if (a.masked) return padded ? launch_forward_hdim_masked(a) : launch_forward_masked(a);
    if (!a.split && uses_key_split(a.B, a.H, a.Nq, a.Nk, a.d, a.causal)) return launch_forward_ks(a);
    if (padded) return launch_forward_hdim(a);
    return launch_variant<false, false>(a);
}

}  // namespace fa
