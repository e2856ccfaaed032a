// PD-transition scan: backward launchers (summary and main pass; kernels in pd.hpp).
#include "pd.hpp"

namespace ssm {

template <typename T, bool DENSE>
hipError_t pd_bwd_t(const PDParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.G + 15) / 16, p.B * p.H);
    // the main backward keeps the generic state count: specialised to 16 its
    // register allocation exceeds the three-waves-per-SIMD budget and spills
    if (summary) {
        if (p.N == 16) pd_bwd_kernel<T, true, 16, -1, DENSE><<<grid, 256, 0, st>>>(p);
        else pd_bwd_kernel<T, true, 0, -1, DENSE><<<grid, 256, 0, st>>>(p);
    } else if (p.glogits) {
        return launch_pd_bwd_ste(p, st);
    } else {
        pd_bwd_kernel<T, false, 0, -1, DENSE><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_pd_bwd(const PDParams& p, bool summary, hipStream_t st) {
    if (p.dense) return p.dtype == 0 ? pd_bwd_t<float, true>(p, summary, st) : pd_bwd_t<bf16_t, true>(p, summary, st);
    return p.dtype == 0 ? pd_bwd_t<float, false>(p, summary, st) : pd_bwd_t<bf16_t, false>(p, summary, st);
}

}  // namespace ssm
