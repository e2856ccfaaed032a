// Issue-rate probes of the VALU instruction classes the scan kernels are built
// from (fp32 FMA and multiply, v_exp_f32, DPP-fused FMA, the cross-row
// permlane swaps), measured on the device at a chosen number of waves per
// SIMD.  They give the measured arithmetic ceiling the roofline divides by.
// Each lane runs `chains` independent dependency chains of one instruction
// class; nothing is read from memory, and one guarded store keeps the chains
// alive.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

// kind: 0 v_fma_f32 (VOP3: the chain value is a multiplicand), 1 v_mul_f32,
// 2 v_exp_f32, 3 v_fmac_f32 with a row_shr:1 DPP source, 4 v_permlane32_swap,
// 5 v_permlane16_swap, 6 v_add_f32, 7 v_fmac_f32 (VOP2: the chain value is the
// addend, which the instruction overwrites)
template <int KIND, int CH>
__global__ __launch_bounds__(64) void roof_kernel(float* __restrict__ out, int iters, float seed) {
    float v[CH], x[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        v[c] = seed + 1e-3f * (float)(threadIdx.x + 7 * c);
        x[c] = 0.5f + 1e-4f * (float)c * seed;
    }
    const float m = 0.999f + 1e-7f * seed, k = 1e-3f * seed;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if constexpr (KIND == 0) {
#pragma unroll
                for (int c = 0; c < CH; ++c) v[c] = fmaf(v[c], m, k);
            } else if constexpr (KIND == 1) {
#pragma unroll
                for (int c = 0; c < CH; ++c) v[c] = v[c] * m;
            } else if constexpr (KIND == 2) {
#pragma unroll
                for (int c = 0; c < CH; ++c) v[c] = __builtin_amdgcn_exp2f(-v[c]);
            } else if constexpr (KIND == 3) {
                // CH = 4 chains in one block: every DPP read is three instructions after the
                // write of its source, which covers the two wait states a DPP read needs (only
                // the very first read may see a stale value, which a rate probe ignores)
                static_assert(CH == 4, "dpp probe runs four chains");
                asm volatile("v_fmac_f32_dpp %0, %0, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                             "v_fmac_f32_dpp %1, %1, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                             "v_fmac_f32_dpp %2, %2, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                             "v_fmac_f32_dpp %3, %3, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
                             : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])
                             : "v"(m));
            } else if constexpr (KIND == 4 || KIND == 5) {
#pragma unroll
                for (int c = 0; c + 1 < CH; c += 2) {
                    auto s = KIND == 4 ? __builtin_amdgcn_permlane32_swap(__float_as_int(v[c]), __float_as_int(v[c + 1]),
                                                                          false, false)
                                       : __builtin_amdgcn_permlane16_swap(__float_as_int(v[c]), __float_as_int(v[c + 1]),
                                                                          false, false);
                    v[c] = __int_as_float(s[0]);
                    v[c + 1] = __int_as_float(s[1]);
                }
            } else if constexpr (KIND == 7) {
#pragma unroll
                for (int c = 0; c < CH; ++c) v[c] = fmaf(x[c], m, v[c]);
            } else {
#pragma unroll
                for (int c = 0; c < CH; ++c) v[c] = v[c] + k;
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += v[c];
    if (s == 1234.5678f) out[blockIdx.x * 64 + threadIdx.x] = s;   // never true for these chains
}

// Instructions per lane of one launch: iters * 8 * (instructions per unrolled step).
double roof_instrs_per_lane(int kind, int chains, int iters) {
    const int per = (kind == 4 || kind == 5) ? chains / 2 : chains;
    return (double)iters * 8.0 * per;
}

hipError_t launch_roof(int kind, int chains, int waves, int iters, float* out, hipStream_t st) {
    const dim3 grid((unsigned)waves), block(64);
#define SSM_ROOF(K, C) roof_kernel<K, C><<<grid, block, 0, st>>>(out, iters, 1.0f)
    if (chains == 4) {
        switch (kind) {
            case 0: SSM_ROOF(0, 4); break;
            case 1: SSM_ROOF(1, 4); break;
            case 2: SSM_ROOF(2, 4); break;
            case 3: SSM_ROOF(3, 4); break;
            case 4: SSM_ROOF(4, 4); break;
            case 5: SSM_ROOF(5, 4); break;
            case 6: SSM_ROOF(6, 4); break;
            default: return hipErrorInvalidValue;
        }
    } else if (chains == 8) {
        switch (kind) {
            case 0: SSM_ROOF(0, 8); break;
            case 1: SSM_ROOF(1, 8); break;
            case 2: SSM_ROOF(2, 8); break;
            case 4: SSM_ROOF(4, 8); break;
            case 5: SSM_ROOF(5, 8); break;
            case 6: SSM_ROOF(6, 8); break;
            case 7: SSM_ROOF(7, 8); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
#undef SSM_ROOF
    return hipGetLastError();
}

}  // namespace ssm
