// PD-transition scan: forward launchers (summary and main pass; kernels in pd.hpp).
#include "pd.hpp"

namespace ssm {

template <typename T, bool DENSE>
hipError_t pd_fwd_t(const PDParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.G + 15) / 16, p.B * p.H);
    if (p.N == 16) {
        if (summary) pd_fwd_kernel<T, true, 16, DENSE><<<grid, 256, 0, st>>>(p);
        else pd_fwd_kernel<T, false, 16, DENSE><<<grid, 256, 0, st>>>(p);
    } else {
        if (summary) pd_fwd_kernel<T, true, 0, DENSE><<<grid, 256, 0, st>>>(p);
        else pd_fwd_kernel<T, false, 0, DENSE><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_pd_fwd(const PDParams& p, bool summary, hipStream_t st) {
    if (p.dense) return p.dtype == 0 ? pd_fwd_t<float, true>(p, summary, st) : pd_fwd_t<bf16_t, true>(p, summary, st);
    return p.dtype == 0 ? pd_fwd_t<float, false>(p, summary, st) : pd_fwd_t<bf16_t, false>(p, summary, st);
}

}  // namespace ssm
