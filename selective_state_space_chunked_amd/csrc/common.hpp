// Device helpers for the gfx950 scan kernels: element conversion, DPP lane
// moves inside 16-lane rows, the affine-operator row scans and the
// transpose-reductions used to sum per-lane partials across lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

// ---------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);  // keep NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                           // nearest even
    return (bf16_t)(u >> 16);
}

// Load KPL consecutive elements starting at p (element index), as float.
// `vec` selects 16-byte vector loads; the caller guarantees alignment then.
template <int KPL>
__device__ __forceinline__ void load_run(const float* __restrict__ p, float (&v)[KPL], bool vec) {
    if (vec) {
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q) {
            float4 w = *reinterpret_cast<const float4*>(p + 4 * q);
            v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) v[j] = p[j];
    }
}
template <int KPL>
__device__ __forceinline__ void load_run(const bf16_t* __restrict__ p, float (&v)[KPL], bool vec) {
    if (vec && (KPL % 8) == 0) {
#pragma unroll
        for (int q = 0; q < KPL / 8; ++q) {
            uint4 w = *reinterpret_cast<const uint4*>(p + 8 * q);
            uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[8 * q + 2 * e] = __uint_as_float(ws[e] << 16);
                v[8 * q + 2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) v[j] = to_f32(p[j]);
    }
}
// Masked variant: elements with index >= n read as 0.
template <typename T, int KPL>
__device__ __forceinline__ void load_run_masked(const T* __restrict__ p, float (&v)[KPL], int n) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) v[j] = (j < n) ? to_f32(p[j]) : 0.0f;
}

template <int KPL>
__device__ __forceinline__ void store_run(float* __restrict__ p, const float (&v)[KPL], bool vec, int n) {
    if (vec && n >= KPL) {
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q)
            *reinterpret_cast<float4*>(p + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (j < n) p[j] = v[j];
    }
}
template <int KPL>
__device__ __forceinline__ void store_run(bf16_t* __restrict__ p, const float (&v)[KPL], bool vec, int n) {
    if (vec && n >= KPL && (KPL % 8) == 0) {
#pragma unroll
        for (int q = 0; q < KPL / 8; ++q) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)from_f32<bf16_t>(v[8 * q + 2 * e]) |
                       ((uint32_t)from_f32<bf16_t>(v[8 * q + 2 * e + 1]) << 16);
            *reinterpret_cast<uint4*>(p + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j)
            if (j < n) p[j] = from_f32<bf16_t>(v[j]);
    }
}

// ---------------------------------------------------------------------------
// DPP moves (gfx9 encodings).  Lanes whose source is outside their 16-lane
// row, or masked off, receive `old`.
// ---------------------------------------------------------------------------
#define SSM_DPP_ROW_SHL(n) (0x100 + (n))
#define SSM_DPP_ROW_SHR(n) (0x110 + (n))
#define SSM_DPP_ROW_ROR(n) (0x120 + (n))
#define SSM_DPP_ROW_MIRROR 0x140
#define SSM_DPP_ROW_HALF_MIRROR 0x141
#define SSM_DPP_ROW_BCAST(n) (0x150 + (n))  // row_newbcast: lane n of each row to the row
#define SSM_DPP_QUAD(a, b, c, d) ((a) | ((b) << 2) | ((c) << 4) | ((d) << 6))

template <int CTRL, int ROWMASK = 0xf, int BANKMASK = 0xf>
__device__ __forceinline__ float dpp(float old, float src) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                      ROWMASK, BANKMASK, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int old, int src) {
    return __builtin_amdgcn_update_dpp(old, src, CTRL, 0xf, 0xf, false);
}

// Broadcast lane `n` (compile-time) of each 16-lane row to the whole row.
template <int n>
__device__ __forceinline__ float row_bcast(float v) { return dpp<SSM_DPP_ROW_BCAST(n)>(0.0f, v); }

// Lane n of each row to the whole row, for an n that is a constant once the
// caller's loop is fully unrolled (the switch then folds to one DPP move).
__device__ __forceinline__ float bcast16(float v, int n) {
    switch (n) {
        case 0: return row_bcast<0>(v);   case 1: return row_bcast<1>(v);
        case 2: return row_bcast<2>(v);   case 3: return row_bcast<3>(v);
        case 4: return row_bcast<4>(v);   case 5: return row_bcast<5>(v);
        case 6: return row_bcast<6>(v);   case 7: return row_bcast<7>(v);
        case 8: return row_bcast<8>(v);   case 9: return row_bcast<9>(v);
        case 10: return row_bcast<10>(v); case 11: return row_bcast<11>(v);
        case 12: return row_bcast<12>(v); case 13: return row_bcast<13>(v);
        case 14: return row_bcast<14>(v); default: return row_bcast<15>(v);
    }
}

// Runtime lane index version (for loops that are not unrolled).
__device__ __forceinline__ float row_bcast_rt(float v, int n) {
    int lane = threadIdx.x & 63;
    int src = (lane & ~15) | n;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// Sum over the 16 lanes of each row; every lane receives the row total.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<SSM_DPP_QUAD(1, 0, 3, 2)>(0.0f, v);
    v += dpp<SSM_DPP_QUAD(2, 3, 0, 1)>(0.0f, v);
    v += dpp<SSM_DPP_ROW_HALF_MIRROR>(0.0f, v);
    v += dpp<SSM_DPP_ROW_MIRROR>(0.0f, v);
    return v;
}

// Inclusive scan, inside each 16-lane row from lane 0 upward, of the affine
// maps f_i(h) = P_i h + S_i under composition (later lane applied last):
// afterwards (P, S) of lane i describe f_i o ... o f_0.
//
// Each of the four levels is two DPP-fused VALU instructions:
//   S_i += S_{i-k} * P_i   (v_fmac_f32 with a row_shr:k source)
//   P_i  = P_{i-k} * P_i   (v_mul_f32 with a row_shr:k source)
// Lanes whose source falls outside the row are not written (bound_ctrl off),
// which leaves lanes i < k unchanged as the scan requires.  A DPP read of a
// VGPR needs two wait states after the VALU write of that VGPR; the s_nop 1
// before every level provides them (the asm block is opaque to the
// compiler's hazard recogniser).
#define SSM_ASM_SCAN_LEVEL(DIR, K)                                               \
    "s_nop 1\n\t"                                                                \
    "v_fmac_f32_dpp %1, %1, %0 " DIR ":" #K " row_mask:0xf bank_mask:0xf\n\t"    \
    "v_mul_f32_dpp %0, %0, %0 " DIR ":" #K " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_scan_affine_up(float& P, float& S) {
    asm volatile(SSM_ASM_SCAN_LEVEL("row_shr", 1) SSM_ASM_SCAN_LEVEL("row_shr", 2)
                 SSM_ASM_SCAN_LEVEL("row_shr", 4) SSM_ASM_SCAN_LEVEL("row_shr", 8)
                 : "+v"(P), "+v"(S));
}
// Inclusive scan from lane 15 downward (lane i composes lanes i..15, lane i
// applied last): used by the reverse-time adjoint recurrence.
__device__ __forceinline__ void row_scan_affine_down(float& P, float& S) {
    asm volatile(SSM_ASM_SCAN_LEVEL("row_shl", 1) SSM_ASM_SCAN_LEVEL("row_shl", 2)
                 SSM_ASM_SCAN_LEVEL("row_shl", 4) SSM_ASM_SCAN_LEVEL("row_shl", 8)
                 : "+v"(P), "+v"(S));
}
#undef SSM_ASM_SCAN_LEVEL
// Both scans at once, interleaved: (P, S) upward, (Q, R) downward.  Every DPP
// read is at least three instructions after the write of its source, so only
// the entry needs wait states.
#define SSM_ASM_SCAN2_LEVEL(K)                                                   \
    "v_fmac_f32_dpp %1, %1, %0 row_shr:" #K " row_mask:0xf bank_mask:0xf\n\t"    \
    "v_fmac_f32_dpp %3, %3, %2 row_shl:" #K " row_mask:0xf bank_mask:0xf\n\t"    \
    "v_mul_f32_dpp %0, %0, %0 row_shr:" #K " row_mask:0xf bank_mask:0xf\n\t"     \
    "v_mul_f32_dpp %2, %2, %2 row_shl:" #K " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void row_scan_affine_updown(float& P, float& S, float& Q, float& R) {
    asm volatile("s_nop 1\n\t" SSM_ASM_SCAN2_LEVEL(1) SSM_ASM_SCAN2_LEVEL(2)
                 SSM_ASM_SCAN2_LEVEL(4) SSM_ASM_SCAN2_LEVEL(8)
                 : "+v"(P), "+v"(S), "+v"(Q), "+v"(R));
}
#undef SSM_ASM_SCAN2_LEVEL

// Exclusive prefix sum within each 16-lane row (lane 0 gets 0).
__device__ __forceinline__ float row_excl_sum_up(float v) {
    float s = v;
    s += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, s);
    return s - v;
}
// Exclusive suffix sum within each row (lane 15 gets 0).
__device__ __forceinline__ float row_excl_sum_down(float v) {
    float s = v;
    s += dpp<SSM_DPP_ROW_SHL(1)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHL(2)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHL(4)>(0.0f, s);
    s += dpp<SSM_DPP_ROW_SHL(8)>(0.0f, s);
    return s - v;
}

// ---------------------------------------------------------------------------
// Transpose-reductions: every lane holds V partial values v[0..V-1]; after the
// call, lane i of each group holds the sum over the group's lanes of slot i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// one halving level inside a 16-lane row, pairing lanes that differ in the bit
// selected by the DPP pattern; `hi` = this lane keeps the upper slot.
template <int CTRL>
__device__ __forceinline__ float pair_level(float lo, float up, bool hi) {
    float keep = hi ? up : lo;
    float send = hi ? lo : up;
    return keep + dpp<CTRL>(0.0f, send);
}

// 16 slots across the 16 lanes of each row: lane i returns sum_lanes v[i].
__device__ __forceinline__ float row_transpose_sum16(const float (&v)[16]) {
    const int l = lane_id() & 15;
    float w[8], z[4], q[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = pair_level<SSM_DPP_ROW_ROR(8)>(v[k], v[k + 8], (l & 8) != 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] = pair_level<SSM_DPP_ROW_HALF_MIRROR>(w[k], w[k + 4], (l & 4) != 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) q[k] = pair_level<SSM_DPP_QUAD(2, 3, 0, 1)>(z[k], z[k + 2], (l & 2) != 0);
    return pair_level<SSM_DPP_QUAD(1, 0, 3, 2)>(q[0], q[1], (l & 1) != 0);
}

// 64 slots across the 64 lanes of a wave: lane i returns sum_lanes v[i].
__device__ __forceinline__ float wave_transpose_sum64(float (&v)[64]) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(v[k]), __float_as_int(v[k + 32]), false, false);
        v[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(v[k]), __float_as_int(v[k + 16]), false, false);
        v[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
    }
    float w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k] = v[k];
    return row_transpose_sum16(w);
}

// 32 slots across the 64 lanes of a wave: lanes 2i and 2i+1 return the sum
// over all lanes of slot i.
__device__ __forceinline__ float wave_transpose_sum32(float (&v)[32]) {
    const int l = lane_id() & 15;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(v[k]), __float_as_int(v[k + 16]), false, false);
        v[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        auto s = __builtin_amdgcn_permlane16_swap(__float_as_int(v[k]), __float_as_int(v[k + 8]), false, false);
        v[k] = __int_as_float(s[0]) + __int_as_float(s[1]);
    }
    float w[4], z[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = pair_level<SSM_DPP_ROW_ROR(8)>(v[k], v[k + 4], (l & 8) != 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) z[k] = pair_level<SSM_DPP_ROW_HALF_MIRROR>(w[k], w[k + 2], (l & 4) != 0);
    float q = pair_level<SSM_DPP_QUAD(2, 3, 0, 1)>(z[0], z[1], (l & 2) != 0);
    return q + dpp<SSM_DPP_QUAD(1, 0, 3, 2)>(0.0f, q);
}

// ---------------------------------------------------------------------------
// fp64 lane moves and transpose-reduction (both 32-bit words move together)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
template <bool WIDE>
__device__ __forceinline__ void permswap_d(double& x, double& y) {
    const long long bx = __double_as_longlong(x), by = __double_as_longlong(y);
    int xl = (int)(bx & 0xffffffffll), xh = (int)(bx >> 32), yl = (int)(by & 0xffffffffll), yh = (int)(by >> 32);
    if (WIDE) {
        auto l = __builtin_amdgcn_permlane32_swap(xl, yl, false, false);
        auto h = __builtin_amdgcn_permlane32_swap(xh, yh, false, false);
        xl = l[0]; yl = l[1]; xh = h[0]; yh = h[1];
    } else {
        auto l = __builtin_amdgcn_permlane16_swap(xl, yl, false, false);
        auto h = __builtin_amdgcn_permlane16_swap(xh, yh, false, false);
        xl = l[0]; yl = l[1]; xh = h[0]; yh = h[1];
    }
    x = __longlong_as_double(((long long)xh << 32) | (unsigned int)xl);
    y = __longlong_as_double(((long long)yh << 32) | (unsigned int)yl);
}
template <int CTRL>
__device__ __forceinline__ double pair_level_d(double lo, double up, bool hi) {
    const double keep = hi ? up : lo;
    const double send = hi ? lo : up;
    return keep + dpp_d<CTRL>(send);
}
// 16 slots across the 64 lanes of a wave, in fp64: lanes 4i..4i+3 return the
// sum over all lanes of slot i.
__device__ __forceinline__ double wave_transpose_sum16_f64(double (&v)[16]) {
    const int l = lane_id() & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        permswap_d<true>(v[k], v[k + 8]);
        v[k] = v[k] + v[k + 8];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        permswap_d<false>(v[k], v[k + 4]);
        v[k] = v[k] + v[k + 4];
    }
    double z[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) z[k] = pair_level_d<SSM_DPP_ROW_ROR(8)>(v[k], v[k + 2], (l & 8) != 0);
    double q = pair_level_d<SSM_DPP_ROW_HALF_MIRROR>(z[0], z[1], (l & 4) != 0);
    q = q + dpp_d<SSM_DPP_QUAD(1, 0, 3, 2)>(q);
    q = q + dpp_d<SSM_DPP_QUAD(2, 3, 0, 1)>(q);
    return q;
}

}  // namespace ssm
