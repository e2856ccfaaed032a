// Fills and copies of small float buffers for the outputs an empty problem (no
// batch rows, channels or steps) still defines: the final state (h0, or zero),
// the adjoint of the initial state (gh_last, or zero) and parameter gradients
// (zero).  A kernel rather than hipMemsetAsync / hipMemcpyAsync keeps the
// entry points capturable in a HIP graph without memset nodes.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

__global__ __launch_bounds__(256) void fill_copy_f32_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                            size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_fill_copy_f32(float* dst, const float* src, size_t n, hipStream_t st) {
    if (!dst || n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
    fill_copy_f32_kernel<<<(unsigned)blocks, 256, 0, st>>>(dst, src, n);
    return hipGetLastError();
}

// zeros of n 16-bit elements (bf16 or half of an f32): the sums over an empty
// channel dimension of a stream gradient of either element type
__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0;
}

hipError_t launch_zero_bytes(void* dst, size_t bytes, hipStream_t st) {
    if (!dst || bytes == 0) return hipSuccess;
    if (bytes % 2) return hipErrorInvalidValue;
    const size_t n = bytes / 2;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
    zero_u16_kernel<<<(unsigned)blocks, 256, 0, st>>>((uint16_t*)dst, n);
    return hipGetLastError();
}

}  // namespace ssm
