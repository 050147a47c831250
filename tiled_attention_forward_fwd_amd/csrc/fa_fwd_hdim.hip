// fa_fwd_hdim.hip -- the attention forward at head dims other than 64 and 128
// (a multiple of 8 up to 128), run by the d = 64 or d = 128 kernel with the
// missing dims held at zero in LDS and registers (fa_fwd_kernel.h with
// PADDED = true). Zero dims add nothing to Q.K^T, and the output dims past d
// are computed but never stored, so the result is that of the head dim d.

#include "fa_fwd_kernel.h"

namespace fa {

hipError_t launch_forward_hdim(const FwdArgs& a) { return launch_variant<false, true>(a); }

}  // namespace fa
