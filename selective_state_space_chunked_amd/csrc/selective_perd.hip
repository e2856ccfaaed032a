// Selective scan forward and backward kernels (selective.hpp), variant with
// per-channel B_t and C_t (Euler input term).
#include "selective.hpp"

namespace ssm {

hipError_t launch_sel_fwd_perd(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    return launch_sel_fwd_var<kVarPerD>(p, dtype, kpl, summary, st);
}
hipError_t launch_sel_bwd_perd(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    return launch_sel_bwd_var<kVarPerD>(p, dtype, kpl, summary, st);
}

}  // namespace ssm
