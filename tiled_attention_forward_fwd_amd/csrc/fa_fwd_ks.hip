// fa_fwd_ks.hip -- launches of the key-split forward for small grids (kernel
// in fa_fwd_ks.h); launch_forward picks it by uses_key_split (fa_launch.h).

#include "fa_fwd_ks.h"

namespace fa {

hipError_t launch_forward_ks(const FwdArgs& a)
{
    const bool padded = a.d != kernel_dim(a.d);
    auto go = [&](auto t, auto dd, auto dc, auto cc, auto pp) -> hipError_t {
        typedef typename decltype(t)::type T;
        constexpr int D = decltype(dd)::value, DC = decltype(dc)::value;
        constexpr bool CAUSAL = decltype(cc)::value, PADDED = decltype(pp)::value;
        if constexpr (DC < D && !PADDED) {
            return hipErrorInvalidValue;  // a computed width below the layout's only comes with padding
        } else {
            return launch_ks_typed<T, D, CAUSAL, PADDED, DC>(a);
        }
    };
    auto by_padded = [&](auto t, auto dd, auto dc, auto cc) -> hipError_t {
        return padded ? go(t, dd, dc, cc, std::true_type()) : go(t, dd, dc, cc, std::false_type());
    };
    auto by_causal = [&](auto t, auto dd, auto dc) -> hipError_t {
        return a.causal ? by_padded(t, dd, dc, std::true_type()) : by_padded(t, dd, dc, std::false_type());
    };
    auto by_compute = [&](auto t, auto dd) -> hipError_t {
        constexpr int D = decltype(dd)::value;
        if (compute_dim(a.d) < D) return by_causal(t, dd, std::integral_constant<int, D - 32>());
        return by_causal(t, dd, dd);
    };
    auto by_dim = [&](auto t) -> hipError_t {
        return kernel_dim(a.d) == 64 ? by_compute(t, std::integral_constant<int, 64>())
                                     : by_compute(t, std::integral_constant<int, 128>());
    };
    return a.bf16 ? by_dim(TypeTag<__bf16>()) : by_dim(TypeTag<_Float16>());
}

}  // namespace fa
