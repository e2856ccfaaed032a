// Selective scan forward main pass that also forms the impulse sensitivity
// d y[t_out] / d x and, with s_delta, d y[t_out] / d delta (selective.hpp,
// SENS = 1, 2): Euler input term, B_t and C_t shared by the channels, 16 states.
#include "selective.hpp"

namespace ssm {

template <typename T, int S>
static hipError_t sel_fwd_sens_t(const SelFwdParams& p, int kpl, hipStream_t st) {
    dim3 grid((p.D + 15) / 16, p.B, p.G), block(256);
    switch (kpl) {
        case 4: sel_fwd_kernel<T, 4, 16, false, kVarEuler, S><<<grid, block, 0, st>>>(p); break;
        case 8: sel_fwd_kernel<T, 8, 16, false, kVarEuler, S><<<grid, block, 0, st>>>(p); break;
        case 16: sel_fwd_kernel<T, 16, 16, false, kVarEuler, S><<<grid, block, 0, st>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sel_fwd_sens(const SelFwdParams& p, int dtype, int kpl, hipStream_t st) {
    if (p.N != 16 || p.var != kVarEuler || (p.s == nullptr && p.s_delta == nullptr) || p.send == nullptr)
        return hipErrorInvalidValue;
    if (p.s_delta) return dtype == 0 ? sel_fwd_sens_t<float, 2>(p, kpl, st) : sel_fwd_sens_t<bf16_t, 2>(p, kpl, st);
    return dtype == 0 ? sel_fwd_sens_t<float, 1>(p, kpl, st) : sel_fwd_sens_t<bf16_t, 1>(p, kpl, st);
}

}  // namespace ssm
