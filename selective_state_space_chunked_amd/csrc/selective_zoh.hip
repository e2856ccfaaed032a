// Selective scan forward and backward kernels (selective.hpp), variant with
// the zero-order-hold input term (B_t, C_t shared by the channels).
#include "selective.hpp"

namespace ssm {

hipError_t launch_sel_fwd_zoh(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    return launch_sel_fwd_var<kVarZoh>(p, dtype, kpl, summary, st);
}
hipError_t launch_sel_bwd_zoh(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    return launch_sel_bwd_var<kVarZoh>(p, dtype, kpl, summary, st);
}

}  // namespace ssm
