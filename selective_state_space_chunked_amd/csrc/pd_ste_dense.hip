// PD-transition scan: main backward pass with the straight-through gradient
// of the selection scores, dense (B,H,L,N) streams (kernels in pd.hpp; the two layouts are
// separate translation units so they compile in parallel).
#include "pd.hpp"

namespace ssm {

template <typename T>
static hipError_t pd_bwd_ste_t(const PDParams& p, hipStream_t st) {
    dim3 grid((p.G + 15) / 16, p.B * p.H);
    if (p.K <= 16) pd_bwd_kernel<T, false, 0, 16, true><<<grid, 256, 0, st>>>(p);
    else if (std::is_same<T, float>::value) pd_bwd_kernel<T, false, 0, 0, true><<<grid, 256, 0, st>>>(p);
    else return hipErrorInvalidValue;   // rejected on the host before: the raw gw needs fp32 storage
    return hipGetLastError();
}
hipError_t launch_pd_bwd_ste_dense(const PDParams& p, hipStream_t st) {
    return p.dtype == 0 ? pd_bwd_ste_t<float>(p, st) : pd_bwd_ste_t<bf16_t>(p, st);
}

}  // namespace ssm
