// fa_fwd_hdim_masked.hip -- padding lengths and sliding windows at head dims
// other than 64 and 128 (fa_fwd_kernel.h with MASKS = true, PADDED = true).

#include "fa_fwd_kernel.h"

namespace fa {

hipError_t launch_forward_hdim_masked(const FwdArgs& a) { return launch_variant<true, true>(a); }

}  // namespace fa
