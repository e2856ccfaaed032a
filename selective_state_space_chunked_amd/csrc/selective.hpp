// Diagonal real selective scan on gfx950, forward and backward kernels:
// a_t[n] = exp(delta_t A[d,n]), input term b_t[n] = delta_t x_t B_t[n] (Euler)
// or (exp(delta_t A[d,n]) - 1) / A[d,n] x_t B_t[n] (zero-order hold), and
// y_t = sum_n C_t[n] h_t[n] (Mamba-style selection and discretisation, lpnh.cn
// "S3M" page, section 1.1).
//
// Work mapping.  A workgroup of 256 lanes is 16 rows of 16 lanes.  Row r owns
// channel d = 16*blockIdx.x + r of batch blockIdx.y; blockIdx.z is a segment
// of consecutive tiles.  A tile is TILE = 16*KPL consecutive steps; lane l of a
// row owns steps l*KPL .. l*KPL+KPL-1 of the tile.  The state index n is a loop
// inside the lane, so sums over n (y, the delta and x gradients) stay in
// registers.  Per-state quantities of a row (A[d,n], the carried state) live
// in lane n of that row and are broadcast with DPP row_newbcast.
//
// Per tile and state n (the three phases of the Flash PD-SSM page's
// "Hardwarebewusste Implementierung", re-mapped onto a 16-lane DPP row):
//   A: every lane folds its KPL steps into one affine map (P, S) with
//      P = prod a = exp2(A2n * sum delta) and S = local state from zero;
//   B: a 4-level DPP scan composes the lane maps across the row; the tile's
//      carry-in comes from the previous tile (sequential within a segment) or,
//      for the first tile of a segment, from a separate segment-combine pass;
//   C: each lane re-runs its KPL steps from its exact entering state and
//      accumulates C_t[n] h_t[n] into y.
// B_t and C_t shared by the channels are staged once per tile in LDS for all
// 16 rows, transposed to [n][t] with 4 floats of padding after every lane's
// run so the 16-byte LDS reads of a row hit distinct banks; per-channel B_t,
// C_t are read by each row from its own slice.  Every streamed tensor is a
// strided view: (b, d) rows at b * s[0] + d * s[1], steps contiguous.
//
// Three variants (template VAR), each compiled in its own translation unit:
// Euler with shared B/C, Euler with per-channel B/C, ZOH with shared B/C.
#pragma once
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// backward workgroup: 32 rows of 16 lanes (channels 32*blockIdx.x ...)
constexpr int kBwdRows = 32;
constexpr int kBwdThreads = 16 * kBwdRows;
// Rows of a wave whose gB/gC products are summed in registers (permlane
// swaps) before the sum over the workgroup's rows in LDS: 1, 2 or 4.
constexpr int kPresum = 4;

// State index of the loop over n: compile-time (fully unrolled loop, DPP
// row_newbcast) or runtime (generic state counts, ds_bpermute broadcast).
template <int NC> struct CState {
    static constexpr int n = NC;
    __device__ __forceinline__ float bc(float v) const { return row_bcast<NC>(v); }
};
struct RState {
    int n;
    __device__ __forceinline__ float bc(float v) const { return row_bcast_rt(v, n); }
};
template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < E) {
        f(CState<I>{});
        static_for<I + 1, E>(f);
    }
}
// Run body(state) for n = 0..N-1: NT = 16 unrolls with compile-time lanes.
template <int NT, typename F>
__device__ __forceinline__ void for_states(int N, F&& body) {
    const int n_end = NT ? NT : N;
#pragma unroll 1
    for (int n = 0; n < n_end; ++n) body(RState{n});
}

template <int KPL> struct TileGeom {
    static constexpr int TILE = 16 * KPL;
    static constexpr int SEG = KPL + 4;          // a lane's run plus padding, in floats
    static constexpr int LDSW = 16 * SEG + 4;    // one state's row; +4 spreads the rows over banks
    __device__ static int idx(int n, int tt) { return n * LDSW + (tt / KPL) * SEG + (tt % KPL); }
};

// Stage a (TILE x N) block of a (B,L,N) tensor (element (b, t, n) at
// b * sb + t * sl + n) into LDS as float [n][t'].  Steps beyond L read as
// zero.  NT = 16: one thread per step row, 16-byte loads when `vec` (rows
// 16-byte aligned).
template <typename T, int KPL, int NT, int THREADS = 256>
__device__ __forceinline__ void stage_tile(float* __restrict__ dst, const T* __restrict__ src, int b, int t0,
                                           int L, int N, int64_t sb, int64_t sl, bool vec) {
    using G = TileGeom<KPL>;
    if constexpr (NT == 16) {
        for (int tt = threadIdx.x; tt < G::TILE; tt += THREADS) {
            const int t = t0 + tt;
            float v[16];
            if (t < L) load_run<16>(src + b * sb + t * sl, v, vec);
            else {
#pragma unroll
                for (int n = 0; n < 16; ++n) v[n] = 0.0f;
            }
            const int base = (tt / KPL) * G::SEG + (tt % KPL);
#pragma unroll
            for (int n = 0; n < 16; ++n) dst[n * G::LDSW + base] = v[n];
        }
    } else {
        const int total = G::TILE * N;
        for (int e = threadIdx.x; e < total; e += THREADS) {
            const int tt = e / N, n = e - tt * N;
            const int t = t0 + tt;
            float v = 0.0f;
            if (t < L) v = to_f32(src[b * sb + t * sl + n]);
            dst[G::idx(n, tt)] = v;
        }
    }
}

// Stage states [nb, ne) of a (TILE x N) block into rows 0 .. ne-nb-1 of dst.
// NT = 16 (halves of 8 states): one thread per step, 8 contiguous values.
template <typename T, int KPL, int NT, int NH, int THREADS = 256>
__device__ __forceinline__ void stage_states(float* __restrict__ dst, const T* __restrict__ src, int b, int t0,
                                             int L, int N, int nb, int ne, int64_t sb, int64_t sl, bool vec) {
    using G = TileGeom<KPL>;
    if constexpr (NT == 16) {
        for (int tt = threadIdx.x; tt < G::TILE; tt += THREADS) {
            const int t = t0 + tt;
            float v[NH];
            if (t < L) load_run<NH>(src + b * sb + t * sl + nb, v, vec);
            else {
#pragma unroll
                for (int n = 0; n < NH; ++n) v[n] = 0.0f;
            }
            const int base = (tt / KPL) * G::SEG + (tt % KPL);
#pragma unroll
            for (int n = 0; n < NH; ++n) dst[n * G::LDSW + base] = v[n];
        }
    } else {
        const int cnt = ne - nb, total = G::TILE * cnt;
        for (int e = threadIdx.x; e < total; e += THREADS) {
            const int tt = e / cnt, n = e - tt * cnt;
            const int t = t0 + tt;
            float v = 0.0f;
            if (t < L) v = to_f32(src[b * sb + t * sl + nb + n]);
            dst[G::idx(n, tt)] = v;
        }
    }
}

// Step sizes from the projection output (S3M page, sections 1.1 and 4.1: the
// discretisation takes delta = softplus(projection(x)), merged into the scan
// kernel): log(1 + e^v), exactly v above 20 (e^-20 is below half an ulp).
__device__ __forceinline__ float softplus_f(float v) { return v > 20.0f ? v : log1pf(expf(v)); }
__device__ __forceinline__ float step_xform(float z, float bias, int softplus) {
    const float v = z + bias;
    return softplus ? softplus_f(v) : v;
}
// d delta / d z = sigmoid(z + bias) = 1 - e^-delta (from the step size itself)
__device__ __forceinline__ float step_xform_grad(float delta, int softplus) {
    return softplus ? -expm1f(-delta) : 1.0f;
}

// A lane's run of step sizes, with the projection-output transform applied;
// steps past the end stay 0 (identity steps).
template <typename T, int KPL>
__device__ __forceinline__ void load_steps(const T* __restrict__ p, float (&dl)[KPL], int nval, bool vec,
                                           const StepXform& f, int d) {
    if (nval >= KPL) load_run<KPL>(p, dl, vec);
    else load_run_masked<T, KPL>(p, dl, nval);
    if (f.bias != nullptr || f.softplus) {   // uniform
        const float bias = f.bias ? f.bias[d] : 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) dl[j] = j < nval ? step_xform(dl[j], bias, f.softplus) : 0.0f;
    }
}

// State n of a lane's run of a per-channel B_t or C_t: p points at (t = the
// lane's first step, n); consecutive steps are sl apart; steps past the end
// read as zero.
template <typename T, int KPL>
__device__ __forceinline__ void load_col(const T* __restrict__ p, int64_t sl, int nval, float (&v)[KPL]) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) v[j] = j < nval ? to_f32(p[j * sl]) : 0.0f;
}

// Zero-order-hold input coefficient (S3M page, section 1.1): b_t = coef * x_t
// B_t with coef = (e^z - 1) / A for z = delta A, a = e^z.  For |z| < 1/4 the
// series delta (1 + z/2 (1 + z/3 (1 + z/4 (1 + z/5 (1 + z/6))))) (truncation
// below 5e-8 relative, no cancellation, exactly delta at A = 0); beyond it
// (a - 1) / A, whose rounding error is below 1e-6 relative there.
__device__ __forceinline__ float zoh_coef(float dl, float z, float a, float invA) {
    const float ser =
        dl * fmaf(z * 0.5f, fmaf(z * (1.0f / 3.0f), fmaf(z * 0.25f, fmaf(z * 0.2f, fmaf(z, 1.0f / 6.0f, 1.0f), 1.0f), 1.0f), 1.0f), 1.0f);
    return fabsf(z) < 0.25f ? ser : (a - 1.0f) * invA;
}
// d coef / d A = delta^2 phi'(z), phi(z) = (e^z - 1) / z, phi'(z) = sum_m (m+1) z^m / (m+2)!
// (series for |z| < 1/4), = (delta a - coef) / A beyond.
__device__ __forceinline__ float zoh_coef_dA(float dl, float z, float a, float coef, float invA) {
    const float ser = dl * dl *
        fmaf(z, fmaf(z, fmaf(z, fmaf(z, fmaf(z, 1.0f / 840.0f, 1.0f / 144.0f), 1.0f / 30.0f), 0.125f), 1.0f / 3.0f), 0.5f);
    return fabsf(z) < 0.25f ? ser : fmaf(dl, a, -coef) * invA;
}
// 1 / A for the ZOH coefficient (unused where A = 0: the series applies there)
__device__ __forceinline__ float zoh_inv(float A) { return A != 0.0f ? 1.0f / A : 0.0f; }

// LDS DMA: every lane of the wave loads 16 bytes from `src` straight into LDS
// at wave_base + 16 * (lane in wave), with no VGPR in between; completion is
// counted by vmcnt like any vector load.
__device__ __forceinline__ void lds_dma16(const void* src, void* wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)wave_base, 16, 0, 0);
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations complete,
// then s_barrier.  Outstanding global loads, stores and LDS DMA keep running
// (__syncthreads would first wait for every one of them to complete).
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// 16-byte LDS store written as assembly.  The compiler cannot tell the LDS DMA
// target from other shared arrays in this kernel and would make every LDS
// store wait for all DMA in flight; these stores never touch the DMA target.
// Completion is covered by the lgkmcnt(0) of lds_barrier.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_store16(float* p, float x, float y, float z, float w) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)p;
    const f32x4 v = {x, y, z, w};
    __asm__ volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
constexpr int kWaitVm0 = 0x0f70;    // s_waitcnt vmcnt(0)
constexpr int kWaitLgkm0 = 0xc07f;  // s_waitcnt lgkmcnt(0)
__device__ __forceinline__ void unpack8_bf16(const uint4& w, float* v) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(ws[e] << 16);
        v[2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
    }
}

template <int KPL>
__device__ __forceinline__ void read_run(const float* __restrict__ s, float (&v)[KPL]) {
#pragma unroll
    for (int q = 0; q < KPL / 4; ++q) {
        float4 w = *reinterpret_cast<const float4*>(s + 4 * q);
        v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
}

// ---------------------------------------------------------------------------
// forward (SUMMARY: segment summaries only, no outputs)
// ---------------------------------------------------------------------------
// The plain main pass stages its B and C tiles eight states at a time (LDS 2 x
// 10.4 KB for KPL 16), so four workgroups fit on a CU next to the 128-VGPR
// budget of four waves per SIMD; the summary and sensitivity passes stage all
// 16 states per round.
constexpr int kFwdStates = 8;

// SENS (main pass, Euler, shared B_t, C_t): also the impulse sensitivity
// s_t = d y[t_out] / d x_t = delta_t sum_n B_t[n] mu_t[n] with the costate
// mu_t[n] = C_out[n] prod_{t < u <= t_out} a_u[n] (PGF page, abstract: reverse
// evolution of the costate).  Within a lane's run it is carried back from the
// run's last step as mu_{j-1} = mu_j a_j with the transitions the scan forms
// anyway; the run's last step takes one exp, 2^(A2 S) with S the sum of delta
// after the run up to t_out (later tiles from send, later lanes by a row sum).
// SENS = 2 adds s_delta_t = d y[t_out] / d delta_t
//   = sum_n mu_t[n] (A[n] a_t[n] h_{t-1}[n] + x_t B_t[n]) = x_t sum_n mu_t B_t + sum_n A[n] mu_{t-1}[n] h_{t-1}[n],
// with mu_t a_t = mu_{t-1} from the same chain and h_{t-1} from the re-run of the states.
template <typename T, int KPL, int NT, bool SUMMARY, int VAR, int SENS = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SENS == 2 ? 2 : SENS ? 3 : 4))) void sel_fwd_kernel(SelFwdParams p) {
    using G = TileGeom<KPL>;
    constexpr int TILE = G::TILE;
    // states staged per round: all 16 where LDS does not limit the occupancy (the summary pass stages
    // no C; the sensitivity pass holds 3 waves per SIMD by its registers anyway)
    constexpr int NH = (SUMMARY || SENS) ? 16 : kFwdStates;
    constexpr bool PERD = VAR == kVarPerD, ZOH = VAR == kVarZoh;
    constexpr bool WD = SENS == 2;
    static_assert(!SENS || (!SUMMARY && VAR == kVarEuler), "the sensitivity rides on the Euler main pass");
    __shared__ __align__(16) float sB[PERD ? 4 : NH * G::LDSW];
    __shared__ __align__(16) float sC[(SUMMARY || PERD) ? 4 : NH * G::LDSW];

    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;
    const T* __restrict__ delta = (const T*)p.delta + ((int64_t)b * p.sdelta[0] + (int64_t)(dc / p.dgrp) * p.sdelta[1]);
    const T* __restrict__ xin = (const T*)p.x + ((int64_t)b * p.sx[0] + (int64_t)dc * p.sx[1]);
    // per-channel B_t, C_t: this row's (b, d) slice, element (t, n) at t * sl + n
    const T* __restrict__ bmrow = (const T*)p.Bm + ((int64_t)b * p.sBm[0] + (int64_t)dc * p.sBm[1]);
    const T* __restrict__ crow = (const T*)p.C + ((int64_t)b * p.sC[0] + (int64_t)dc * p.sC[1]);
    const size_t seq = (size_t)b * p.D + dc;

    float A2 = 0.0f, carry = 0.0f, Pseg = 1.0f, invA = 0.0f, cout = 0.0f;
    if (lane < N) {
        const float Av = p.A[(int64_t)(dc / p.agrp) * p.sA + lane * p.sAn];
        A2 = Av * kLog2e;
        if (ZOH) invA = zoh_inv(Av);
        if (!SUMMARY) {
            if (p.G > 1) carry = p.carry_in[(seq * p.G + g) * N + lane];
            else if (p.h0) carry = p.h0[seq * N + lane];
        }
        if (SENS) cout = to_f32(((const T*)p.C)[(int64_t)b * p.sC[0] + (int64_t)p.t_out * p.sC[2] + lane]);
    }
    const int tile0 = g * p.tiles_per_seg;
    const int tile1 = min(tile0 + p.tiles_per_seg, p.ntiles);
    const bool vec = p.vec != 0, bcvec = p.bc_vec != 0;

    for (int tile = tile0; tile < tile1; ++tile) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * KPL;
        const int nval = L - tl;
        // dx = delta x (Euler); the ZOH form keeps x itself (its coefficient depends on the state)
        float dl[KPL], dx[KPL];
        float xk[WD ? KPL : 1];   // the step-size sensitivity keeps x for its x_t sum_n mu B term
        {
            float xv[KPL];
            load_steps<T, KPL>(delta + tl, dl, nval, vec, p.stepf, dc);
            if (nval >= KPL) load_run<KPL>(xin + tl, xv, vec);
            else load_run_masked<T, KPL>(xin + tl, xv, nval);
#pragma unroll
            for (int j = 0; j < KPL; ++j) dx[j] = ZOH ? xv[j] : dl[j] * xv[j];
            if constexpr (WD) {
#pragma unroll
                for (int j = 0; j < KPL; ++j) xk[j] = xv[j];
            }
        }
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) dsum += dl[j];
        if (p.tile_dsum) {
            float ts = row_sum(dsum);
            if (act && lane == 0) p.tile_dsum[seq * p.ntiles + tile] = ts;
        }
        if (!SUMMARY && p.ckpt && act && lane < N) p.ckpt[(seq * p.ntiles + tile) * N + lane] = carry;

        float yacc[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) yacc[j] = 0.0f;
        // sensitivity: tiles after t_out's are zero; in t_out's tile only steps up to t_out count
        const bool sens_tile = SENS && t0 <= p.t_out;    // uniform
        const bool tout_tile = SENS && p.t_out < t0 + TILE;
        float sacc[SENS ? KPL : 1], gd[WD ? KPL : 1], sbase = 0.0f;
#pragma unroll
        for (int j = 0; j < (SENS ? KPL : 1); ++j) sacc[j] = 0.0f;
#pragma unroll
        for (int j = 0; j < (WD ? KPL : 1); ++j) gd[j] = 0.0f;
        if (sens_tile) {
            float lsum = dsum;
            if (tout_tile) {
                lsum = 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) lsum += tl + j <= p.t_out ? dl[j] : 0.0f;
            }
            // sum of delta after this lane's run, up to t_out
            sbase = (float)p.send[seq * p.ntiles + tile] + row_excl_sum_down(lsum);
        }

        // the state loop; TOUT: t_out lies inside this tile (sensitivity only)
        auto states = [&](auto tout_c) {
            constexpr bool TOUT = decltype(tout_c)::value;
            for (int nb = 0; nb < N; nb += NH) {
                const int ne = min(nb + NH, N);
                if constexpr (!PERD) {
                    lds_barrier();
                    stage_states<T, KPL, NT, NH>(sB, (const T*)p.Bm, b, t0, L, N, nb, ne, p.sBm[0],
                                                 p.sBm[2], bcvec);
                    if (!SUMMARY)
                        stage_states<T, KPL, NT, NH>(sC, (const T*)p.C, b, t0, L, N, nb, ne, p.sC[0], p.sC[2], bcvec);
                    lds_barrier();
                }
                // the broadcasts for state n+1 are issued while state n runs (lane n+1's
                // carry does not change during step n)
                float A2n_nx = row_bcast_rt(A2, nb), cin_nx = row_bcast_rt(carry, nb);
                float iA_nx = ZOH ? row_bcast_rt(invA, nb) : 0.0f;
#pragma unroll 1
                for (int n = nb; n < ne; ++n) {
                    const int nr = n - nb;   // row of state n in the staged half
                    const float A2n = A2n_nx, cin = cin_nx, iAn = iA_nx;
                    {
                        const int nn = min(n + 1, ne - 1);
                        A2n_nx = row_bcast_rt(A2, nn);
                        cin_nx = row_bcast_rt(carry, nn);
                        if (ZOH) iA_nx = row_bcast_rt(invA, nn);
                    }
                    float bv[KPL], a[KPL], bx[KPL];
                    if constexpr (PERD) load_col<T, KPL>(bmrow + (int64_t)tl * p.sBm[2] + n, p.sBm[2], nval, bv);
                    else read_run<KPL>(sB + nr * G::LDSW + lane * G::SEG, bv);
                    float S = 0.0f;
#pragma unroll
                    for (int j = 0; j < KPL; ++j) {
                        const float z2 = dl[j] * A2n;
                        a[j] = __builtin_amdgcn_exp2f(z2);
                        if constexpr (ZOH) bx[j] = zoh_coef(dl[j], z2 * kLn2, a[j], iAn) * dx[j] * bv[j];
                        else bx[j] = dx[j] * bv[j];
                        S = fmaf(a[j], S, bx[j]);
                    }
                    float P = __builtin_amdgcn_exp2f(dsum * A2n);
                    row_scan_affine_up(P, S);
                    // WD: A[n] mu_{j-1}, used by the re-run below against h_{j-1}
                    float ma[WD ? KPL : 1];
                    if constexpr (SENS) {   // bv is not needed after this
                        const float Cn = row_bcast_rt(cout, n);
                        const float An = A2n * kLn2;
                        if (sens_tile) {
                            // costate at the run's last step, then mu_{j-1} = mu_j a_j
                            float m = Cn * __builtin_amdgcn_exp2f(A2n * sbase);
                            if constexpr (!TOUT) {
#pragma unroll
                                for (int j = KPL - 1; j >= 0; --j) {
                                    sacc[j] = fmaf(bv[j], m, sacc[j]);
                                    m *= a[j];
                                    if constexpr (WD) ma[j] = An * m;
                                }
                            } else {
                                // zero after t_out, C_out at t_out
                                if (tl + KPL - 1 > p.t_out) m = 0.0f;
#pragma unroll
                                for (int j = KPL - 1; j >= 0; --j) {
                                    if (tl + j == p.t_out) m = Cn;
                                    sacc[j] = fmaf(bv[j], m, sacc[j]);
                                    m *= a[j];
                                    if constexpr (WD) ma[j] = An * m;
                                }
                            }
                        }
                    }
                    float newc;
                    if constexpr (SUMMARY) {
                        const float Pt = row_bcast<15>(P), St = row_bcast<15>(S);
                        newc = fmaf(Pt, cin, St);
                        if (lane == n) Pseg *= Pt;
                    } else {
                        const float hend = fmaf(P, cin, S);
                        float h = dpp<SSM_DPP_ROW_SHR(1)>(cin, hend);  // state entering this lane's run
                        newc = row_bcast<15>(hend);
                        float cv[KPL];
                        if constexpr (PERD) load_col<T, KPL>(crow + (int64_t)tl * p.sC[2] + n, p.sC[2], nval, cv);
                        else read_run<KPL>(sC + nr * G::LDSW + lane * G::SEG, cv);
                        if (WD && sens_tile) {
#pragma unroll
                            for (int j = 0; j < KPL; ++j) {
                                gd[j] = fmaf(ma[WD ? j : 0], h, gd[j]);   // h = h_{j-1}
                                h = fmaf(a[j], h, bx[j]);
                                yacc[j] = fmaf(cv[j], h, yacc[j]);
                            }
                        } else {
#pragma unroll
                            for (int j = 0; j < KPL; ++j) {
                                h = fmaf(a[j], h, bx[j]);
                                yacc[j] = fmaf(cv[j], h, yacc[j]);
                            }
                        }
                    }
                    carry = (lane == n) ? newc : carry;
                }
            }
        };
        if (SENS && tout_tile) states(std::true_type{});
        else states(std::false_type{});
        if (!SUMMARY && p.y && act && nval > 0)
            store_run<KPL>((T*)p.y + ((int64_t)b * p.sy[0] + (int64_t)dc * p.sy[1]) + tl, yacc, vec, nval);
        if (SENS && act && nval > 0) {
            float v[KPL];
            if (p.s) {
#pragma unroll
                for (int j = 0; j < KPL; ++j) v[j] = (sens_tile && tl + j <= p.t_out) ? dl[j] * sacc[j] : 0.0f;
                store_run<KPL>((T*)p.s + seq * L + tl, v, vec, nval);
            }
            if constexpr (WD) {
                // d delta / d z times d y / d delta
#pragma unroll
                for (int j = 0; j < KPL; ++j)
                    v[j] = (sens_tile && tl + j <= p.t_out)
                               ? fmaf(xk[j], sacc[j], gd[j]) * step_xform_grad(dl[j], p.stepf.softplus)
                               : 0.0f;
                store_run<KPL>((T*)p.s_delta + seq * L + tl, v, vec, nval);
            }
        }
    }
    if (SUMMARY) {
        if (act && lane < N) {
            p.segP[(seq * p.G + g) * N + lane] = Pseg;
            p.segS[(seq * p.G + g) * N + lane] = carry;
        }
    } else if (p.h_last && g == p.G - 1 && act && lane < N) {
        p.h_last[seq * N + lane] = carry;
    }
}

// ---------------------------------------------------------------------------
// backward.  Reverse over the tiles of a segment.  Per tile and state n: the
// forward is recomputed from the checkpoint (phases A-C as above, states kept
// in registers), then the adjoint nu_t = a_t (C_t gy_t + nu_{t+1}) runs right
// to left with the same lane-fold / DPP-scan structure, seeded by the adjoint
// entering from the next tile (gh_last at the sequence end).
//   lambda_t = C_t gy_t + nu_{t+1},   dLoss/da_t = lambda_t h_{t-1},
//   gdelta_t = sum_n (A lambda a h_{t-1} + lambda x B),  gx_t = delta_t sum_n lambda B,
//   gB_t[n] = sum_d lambda delta x,  gC_t[n] = sum_d gy h_t,  gA = sum_{b,t} lambda a h_{t-1} delta.
// Sums over d (gB, gC) are taken over the 4 rows of each wave with permlane
// swaps, then over the 8 waves in LDS, and written as one partial per
// 32-channel block; a second kernel adds the blocks in order.
// SUMMARY: per segment, the composed adjoint map nu_start = Q nu_end + R.
// bf16 streams with 16-step runs and 16 states: while a tile runs, the next
// tile's delta, x and gy runs and its B and C rows are fetched into LDS by DMA
// (no registers held), and its checkpoint into a register, so a tile starts
// without waiting on HBM.
// ---------------------------------------------------------------------------
template <typename T, int KPL, int NT, bool SUMMARY, bool WA, int VAR>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void sel_bwd_kernel(SelBwdParams p) {
    using G = TileGeom<KPL>;
    constexpr int TILE = G::TILE;
    constexpr int ROWS = kBwdRows;
    constexpr bool PERD = VAR == kVarPerD, ZOH = VAR == kVarZoh;
    __shared__ __align__(16) float sB[(SUMMARY || PERD) ? 4 : 16 * G::LDSW];
    __shared__ __align__(16) float sC[PERD ? 4 : 16 * G::LDSW];
    // Partials of gB and gC for one state after the in-wave pre-sum, laid out
    // like the B/C tiles ([pre-summed row][lane run + 4 pad]); two buffers
    // (state parity) so one barrier per state suffices.  Per-channel B_t, C_t
    // have per-channel gradients: no sum over channels, no LDS.
    constexpr int RB = ROWS / kPresum;
    __shared__ __align__(16) float red[(SUMMARY || PERD) ? 4 : 2 * 2 * RB * G::LDSW];
    // next-tile prefetch: per wave [delta | x | gy][half run][lane], and the raw B, C rows [t][half]
    constexpr bool PF = sizeof(T) == 2 && KPL == 16 && NT == 16 && !SUMMARY && !PERD;
    static_assert(!PF || kBwdThreads == 2 * TILE, "one B row half per thread");
    __shared__ __align__(16) uint4 pfs[PF ? (ROWS / 4) * 3 * 2 * 64 : 1];
    __shared__ __align__(16) uint4 pfbc[PF ? 2 * 2 * TILE : 1];

    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * ROWS + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;
    const T* __restrict__ delta = (const T*)p.delta + ((int64_t)b * p.sdelta[0] + (int64_t)(dc / p.dgrp) * p.sdelta[1]);
    const T* __restrict__ xin = (const T*)p.x + ((int64_t)b * p.sx[0] + (int64_t)dc * p.sx[1]);
    const T* __restrict__ gyin = (const T*)p.gy + ((int64_t)b * p.sgy[0] + (int64_t)dc * p.sgy[1]);
    const T* __restrict__ bmrow = (const T*)p.Bm + ((int64_t)b * p.sBm[0] + (int64_t)dc * p.sBm[1]);
    const T* __restrict__ crow = (const T*)p.C + ((int64_t)b * p.sC[0] + (int64_t)dc * p.sC[1]);
    const size_t seq = (size_t)b * p.D + dc;
    const bool vec = p.vec != 0, bcvec = p.bc_vec != 0;
    const bool wantB = p.partB != nullptr, wantC = p.partC != nullptr;
    // per-channel gradients of B_t and C_t: (B, D, L, N) dense
    T* __restrict__ gbrow = PERD && p.gBm_pd ? (T*)p.gBm_pd + seq * (size_t)L * N : nullptr;
    T* __restrict__ gcrow = PERD && p.gC_pd ? (T*)p.gC_pd + seq * (size_t)L * N : nullptr;

    float A2 = 0.0f, nu = 0.0f, gAacc = 0.0f, Qseg = 1.0f, gbias = 0.0f, invA = 0.0f;
    if (lane < N) {
        const float Av = p.A[(int64_t)(dc / p.agrp) * p.sA + lane * p.sAn];
        A2 = Av * kLog2e;
        if (ZOH) invA = zoh_inv(Av);
        if (!SUMMARY) {
            if (p.G > 1) nu = p.nu_in[(seq * p.G + g) * N + lane];
            else if (p.gh_last) nu = p.gh_last[seq * N + lane];
        }
    }
    const int tile0 = g * p.tiles_per_seg;
    const int tile1 = min(tile0 + p.tiles_per_seg, p.ntiles);
    // prefetch (uniform): aligned rows; every tile but the last of the sequence is whole
    const bool pf = PF && vec && bcvec;
    uint4* pfw = pfs + (tid >> 6) * (3 * 2 * 64);   // this wave's slots
    float hs_nx = 0.0f;                            // checkpoint of the next tile, one ahead
    const size_t ckt = p.ckpt_tiles ? (size_t)p.ckpt_tiles : (size_t)p.ntiles;
    if (!SUMMARY && lane < N) hs_nx = p.ckpt[(seq * ckt + (size_t)(tile1 - 1) * p.ckpt_every) * N + lane];

    for (int tile = tile1 - 1; tile >= tile0; --tile) {
        const int t0 = tile * TILE;
        const bool have = pf && tile != tile1 - 1;   // this tile's streams are in LDS
        if constexpr (!PERD) {
            if (PF && have) __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's DMA has landed
            lds_barrier();
            if (PF && have) {
                // rows of the raw B (threads 0..TILE-1) and C tiles into [n][t'] layout
                const int tt = tid & (TILE - 1);
                const uint4* src = pfbc + (tid >= TILE ? 2 * TILE : 0) + 2 * tt;
                float* dst = tid >= TILE ? sC : sB;
                float v[16];
                unpack8_bf16(src[0], v);
                unpack8_bf16(src[1], v + 8);
                const int base = (tt / KPL) * G::SEG + (tt % KPL);
#pragma unroll
                for (int n = 0; n < 16; ++n) dst[n * G::LDSW + base] = v[n];
            } else {
                if (!SUMMARY) stage_tile<T, KPL, NT, kBwdThreads>(sB, (const T*)p.Bm, b, t0, L, N, p.sBm[0], p.sBm[2], bcvec);
                stage_tile<T, KPL, NT, kBwdThreads>(sC, (const T*)p.C, b, t0, L, N, p.sC[0], p.sC[2], bcvec);
            }
            lds_barrier();
            if (PF && pf && tile > tile0) {   // B and C rows of the next tile: thread i, row i / 2, half i % 2
                const int64_t tn = (int64_t)(t0 - TILE) + (tid >> 1);
                const int h8 = 8 * (tid & 1);
                lds_dma16((const T*)p.Bm + b * p.sBm[0] + tn * p.sBm[2] + h8, pfbc + (tid & ~63));
                lds_dma16((const T*)p.C + b * p.sC[0] + tn * p.sC[2] + h8, pfbc + 2 * TILE + (tid & ~63));
            }
        }

        const int tl = t0 + lane * KPL;
        const int nval = L - tl;
        // dx = delta x (Euler); the ZOH form keeps x itself
        float dl[KPL], dx[KPL], gyv[KPL];
        uint4 xr0 = {0u, 0u, 0u, 0u}, xr1 = {0u, 0u, 0u, 0u};   // prefetched x run, kept for the delta gradient
        {
            float xv[KPL];
            if (PF && have) {
                const int wl = tid & 63;
                const uint4 d0 = pfw[wl], d1 = pfw[64 + wl], g0 = pfw[256 + wl], g1 = pfw[320 + wl];
                xr0 = pfw[128 + wl];
                xr1 = pfw[192 + wl];
                unpack8_bf16(d0, dl);
                unpack8_bf16(d1, dl + 8);
                unpack8_bf16(g0, gyv);
                unpack8_bf16(g1, gyv + 8);
                unpack8_bf16(xr0, xv);
                unpack8_bf16(xr1, xv + 8);
                if (p.stepf.bias != nullptr || p.stepf.softplus) {   // uniform
                    const float bias = p.stepf.bias ? p.stepf.bias[dc] : 0.0f;
#pragma unroll
                    for (int j = 0; j < KPL; ++j) dl[j] = step_xform(dl[j], bias, p.stepf.softplus);
                }
            } else {
                load_steps<T, KPL>(delta + tl, dl, nval, vec, p.stepf, dc);
                if (nval >= KPL) {
                    load_run<KPL>(gyin + tl, gyv, vec);
                    if (!SUMMARY) load_run<KPL>(xin + tl, xv, vec);
                } else {
                    load_run_masked<T, KPL>(gyin + tl, gyv, nval);
                    if (!SUMMARY) load_run_masked<T, KPL>(xin + tl, xv, nval);
                }
            }
            if (PF && pf && tile > tile0) {   // this lane's runs of the next tile
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the slots above have been read
                const int tn = tl - TILE;
                lds_dma16(delta + tn, pfw);
                lds_dma16(delta + tn + 8, pfw + 64);
                lds_dma16(xin + tn, pfw + 128);
                lds_dma16(xin + tn + 8, pfw + 192);
                lds_dma16(gyin + tn, pfw + 256);
                lds_dma16(gyin + tn + 8, pfw + 320);
            }
            // rows past D contribute nothing to the sums over channels
            const float live = act ? 1.0f : 0.0f;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                dx[j] = SUMMARY ? 0.0f : (ZOH ? xv[j] : dl[j] * xv[j]) * live;
                if (!SUMMARY) gyv[j] *= live;
            }
        }
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) dsum += dl[j];
        const float hs = hs_nx;
        if (!SUMMARY && lane < N && tile > tile0) hs_nx = p.ckpt[(seq * ckt + (size_t)(tile - 1) * p.ckpt_every) * N + lane];

        float Gd[KPL], Sb[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) { Gd[j] = 0.0f; Sb[j] = 0.0f; }

        // broadcasts of state n+1 are issued while state n runs (lane n+1's adjoint
        // does not change during step n)
        float A2n_nx = row_bcast_rt(A2, 0), nin_nx = row_bcast_rt(nu, 0), cin_nx = row_bcast_rt(hs, 0);
        float iA_nx = ZOH ? row_bcast_rt(invA, 0) : 0.0f;
        const int n_end = NT ? NT : N;
#pragma unroll 1
        for (int n = 0; n < n_end; ++n) {
            const float A2n = A2n_nx, nin = nin_nx, cin = cin_nx, iAn = iA_nx;
            {
                const int nn = min(n + 1, n_end - 1);
                A2n_nx = row_bcast_rt(A2, nn);
                nin_nx = row_bcast_rt(nu, nn);
                if (!SUMMARY) cin_nx = row_bcast_rt(hs, nn);
                if (ZOH && !SUMMARY) iA_nx = row_bcast_rt(invA, nn);
            }
            float a[KPL], cv[KPL];
            if constexpr (PERD) load_col<T, KPL>(crow + (int64_t)tl * p.sC[2] + n, p.sC[2], nval, cv);
            else read_run<KPL>(sC + n * G::LDSW + lane * G::SEG, cv);
#pragma unroll
            for (int j = 0; j < KPL; ++j) a[j] = __builtin_amdgcn_exp2f(dl[j] * A2n);
            const float P = __builtin_amdgcn_exp2f(dsum * A2n);

            // adjoint lane fold, right to left: nu_j = a_j (c_j + nu_{j+1})
            float R = 0.0f;
#pragma unroll
            for (int j = KPL - 1; j >= 0; --j) R = a[j] * fmaf(cv[j], gyv[j], R);
            float Q = P;
            if constexpr (SUMMARY) {
                row_scan_affine_down(Q, R);
                const float nfirst = fmaf(Q, nin, R);     // adjoint at this lane's first step
                const float newnu = row_bcast<0>(nfirst);
                const float Qt = row_bcast<0>(Q);
                if (lane == n) Qseg *= Qt;
                nu = (lane == n) ? newnu : nu;
            } else {
                // forward lane fold of the recomputed states, scanned together with the adjoint
                const float An = A2n * kLn2;   // A[d, n]
                float bv[KPL], bx[KPL], h[KPL + 1], coef[ZOH ? KPL : 1];
                if constexpr (PERD) load_col<T, KPL>(bmrow + (int64_t)tl * p.sBm[2] + n, p.sBm[2], nval, bv);
                else read_run<KPL>(sB + n * G::LDSW + lane * G::SEG, bv);
                float S = 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    if constexpr (ZOH) {
                        coef[j] = zoh_coef(dl[j], dl[j] * An, a[j], iAn);
                        bx[j] = coef[j] * dx[j] * bv[j];
                    } else {
                        bx[j] = dx[j] * bv[j];
                    }
                    S = fmaf(a[j], S, bx[j]);
                }
                float Pf = P;
                row_scan_affine_updown(Pf, S, Q, R);
                const float nfirst = fmaf(Q, nin, R);     // adjoint at this lane's first step
                const float newnu = row_bcast<0>(nfirst);
                float nnext = dpp<SSM_DPP_ROW_SHL(1)>(nin, nfirst);  // adjoint entering from the right
                const float hend = fmaf(Pf, cin, S);
                h[0] = dpp<SSM_DPP_ROW_SHR(1)>(cin, hend);         // state entering this lane's run
#pragma unroll
                for (int j = 0; j < KPL; ++j) h[j + 1] = fmaf(a[j], h[j], bx[j]);

                float gAl = 0.0f;
                float pB[KPL], pC[KPL];
#pragma unroll
                for (int j = KPL - 1; j >= 0; --j) {
                    const float lam = fmaf(cv[j], gyv[j], nnext);
                    nnext = a[j] * lam;                       // nu_j
                    const float t1 = nnext * h[j];            // lambda_j a_j h_{j-1}
                    Gd[j] = fmaf(An, t1, Gd[j]);
                    if constexpr (ZOH) {
                        // d b / d delta = a x B, d b / d x = coef B, d b / d B = coef x
                        Gd[j] = fmaf(nnext, dx[j] * bv[j], Gd[j]);
                        Sb[j] = fmaf(lam, coef[j] * bv[j], Sb[j]);
                        if constexpr (WA) {
                            const float dcA = zoh_coef_dA(dl[j], dl[j] * An, a[j], coef[j], iAn);
                            gAl = fmaf(t1, dl[j], fmaf(lam * bv[j], dx[j] * dcA, gAl));
                        }
                        pB[j] = lam * (coef[j] * dx[j]);
                    } else {
                        Sb[j] = fmaf(lam, bv[j], Sb[j]);
                        if constexpr (WA) gAl = fmaf(t1, dl[j], gAl);
                        pB[j] = lam * dx[j];
                    }
                    pC[j] = gyv[j] * h[j + 1];
                }
                if constexpr (PERD) {
                    // per-channel gradients of B_t and C_t: written as they are, step by step
                    if (act) {
#pragma unroll
                        for (int j = 0; j < KPL; ++j) {
                            if (j < nval) {
                                const size_t o = (size_t)(tl + j) * N + n;
                                if (gbrow) gbrow[o] = from_f32<T>(pB[j]);
                                if (gcrow) gcrow[o] = from_f32<T>(pC[j]);
                            }
                        }
                    }
                    nu = (lane == n) ? newnu : nu;
                    if constexpr (WA) {
                        const float ga = row_sum(gAl);
                        if (lane == n) gAacc += ga;
                    }
                } else {
                // sum the wave's rows in registers: level 1 adds rows r and r+2 (lanes l, l+32),
                // level 2 rows r and r+1; afterwards a lane holds KPL/kPresum consecutive steps
                // of its lane run, summed over the kPresum rows
                constexpr int CNT = KPL / kPresum;
                if constexpr (kPresum >= 2) {
#pragma unroll
                    for (int j = 0; j < KPL / 2; ++j) {
                        auto sb = __builtin_amdgcn_permlane32_swap(__float_as_int(pB[j]), __float_as_int(pB[j + KPL / 2]),
                                                                   false, false);
                        pB[j] = __int_as_float(sb[0]) + __int_as_float(sb[1]);
                        auto sc = __builtin_amdgcn_permlane32_swap(__float_as_int(pC[j]), __float_as_int(pC[j + KPL / 2]),
                                                                   false, false);
                        pC[j] = __int_as_float(sc[0]) + __int_as_float(sc[1]);
                    }
                }
                if constexpr (kPresum >= 4) {
#pragma unroll
                    for (int j = 0; j < KPL / 4; ++j) {
                        auto sb = __builtin_amdgcn_permlane16_swap(__float_as_int(pB[j]), __float_as_int(pB[j + KPL / 4]),
                                                                   false, false);
                        pB[j] = __int_as_float(sb[0]) + __int_as_float(sb[1]);
                        auto sc = __builtin_amdgcn_permlane16_swap(__float_as_int(pC[j]), __float_as_int(pC[j + KPL / 4]),
                                                                   false, false);
                        pC[j] = __int_as_float(sc[0]) + __int_as_float(sc[1]);
                    }
                }
                float* buf = red + (n & 1) * (2 * RB * G::LDSW);
                {
                    constexpr int GRP = 4 / kPresum;             // pre-summed rows per wave
                    const int q = row & 3, w = row >> 2;
                    const int rb = w * GRP + (q % GRP);
                    float* rB = buf + rb * G::LDSW + lane * G::SEG + (q / GRP) * CNT;
                    float* rC = rB + RB * G::LDSW;
                    if constexpr (PF) {
#pragma unroll
                        for (int k = 0; k < CNT / 4; ++k) {
                            lds_store16(rB + 4 * k, pB[4 * k], pB[4 * k + 1], pB[4 * k + 2], pB[4 * k + 3]);
                            lds_store16(rC + 4 * k, pC[4 * k], pC[4 * k + 1], pC[4 * k + 2], pC[4 * k + 3]);
                        }
                    } else if constexpr (CNT % 4 == 0) {
#pragma unroll
                        for (int k = 0; k < CNT / 4; ++k) {
                            *reinterpret_cast<float4*>(rB + 4 * k) =
                                make_float4(pB[4 * k], pB[4 * k + 1], pB[4 * k + 2], pB[4 * k + 3]);
                            *reinterpret_cast<float4*>(rC + 4 * k) =
                                make_float4(pC[4 * k], pC[4 * k + 1], pC[4 * k + 2], pC[4 * k + 3]);
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < CNT; ++k) { rB[k] = pB[k]; rC[k] = pC[k]; }
                    }
                }
                nu = (lane == n) ? newnu : nu;
                if constexpr (WA) {
                    const float ga = row_sum(gAl);
                    if (lane == n) gAacc += ga;
                }
                if (wantB || wantC) {
                    // the other buffer was last read before the previous state's barrier, so
                    // this single barrier orders both the writes above and the reads below
                    lds_barrier();
                    // one output per thread; each half-wave takes 8 lane runs x 4 steps, whose
                    // words (run * (KPL + 4) + step) fall in 32 distinct banks
                    for (int o = tid; o < 2 * TILE; o += kBwdThreads) {
                        const int which = o / TILE, i = o - which * TILE;
                        const int k = i & 63;
                        const int tt = ((k & 7) + 8 * (k >> 5)) * KPL + 4 * (i >> 6) + ((k >> 3) & 3);
                        const float* src = buf + which * RB * G::LDSW + (tt / KPL) * G::SEG + (tt % KPL);
                        float sum = 0.0f;
#pragma unroll
                        for (int r = 0; r < RB; ++r) sum += src[r * G::LDSW];
                        float* part = which ? p.partC : p.partB;
                        const int t = t0 + tt;
                        if (part && t < L) part[(((size_t)blockIdx.x * p.B + b) * N + n) * L + t] = sum;
                    }
                }
                }
            }
        }
        if (!SUMMARY && act && nval > 0) {
            if (p.gx) {
                float v[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) v[j] = ZOH ? Sb[j] : dl[j] * Sb[j];
                store_run<KPL>((T*)p.gx + ((int64_t)b * p.sgx[0] + (int64_t)dc * p.sgx[1]) + tl, v, vec, nval);
            }
            if (p.gdelta || p.partBias) {
                // gradient w.r.t. delta as given (the projection output when the
                // step sizes are transformed): d delta/d z times d Loss/d delta
                float v[KPL];
                if constexpr (ZOH) {
#pragma unroll
                    for (int j = 0; j < KPL; ++j) v[j] = Gd[j] * step_xform_grad(dl[j], p.stepf.softplus);
                } else {
                    float xv[KPL];
                    if (PF && have) {
                        unpack8_bf16(xr0, xv);
                        unpack8_bf16(xr1, xv + 8);
                    } else if (nval >= KPL) {
                        load_run<KPL>(xin + tl, xv, vec);
                    } else {
                        load_run_masked<T, KPL>(xin + tl, xv, nval);
                    }
#pragma unroll
                    for (int j = 0; j < KPL; ++j)
                        v[j] = fmaf(xv[j], Sb[j], Gd[j]) * step_xform_grad(dl[j], p.stepf.softplus);
                }
                if (p.gdelta) {
                    const int64_t o = (int64_t)b * p.sgdelta[0] + (int64_t)dc * p.sgdelta[1] + tl;
                    if (p.gdelta_f32) store_run<KPL>((float*)p.gdelta + o, v, vec, nval);   // uniform
                    else store_run<KPL>((T*)p.gdelta + o, v, vec, nval);
                }
#pragma unroll
                for (int j = 0; j < KPL; ++j) gbias += j < nval ? v[j] : 0.0f;
            }
        }
    }
    if (SUMMARY) {
        if (act && lane < N) {
            p.segQ[(seq * p.G + g) * N + lane] = Qseg;
            p.segR[(seq * p.G + g) * N + lane] = nu;
        }
        return;
    }
    if (p.partBias) {   // uniform; every lane of the row takes part in the sum
        gbias = row_sum(gbias);
        if (act && lane == 0) p.partBias[((size_t)b * p.G + g) * p.D + dc] = gbias;
    }
    if (act && lane < N) {
        if (p.gh0 && g == 0) p.gh0[seq * N + lane] = nu;
        if (WA) p.partA[(((size_t)b * p.G + g) * p.D + dc) * N + lane] = gAacc;
    }
}

// Launchers of one kernel variant (instantiated by the translation unit that
// compiles that variant).
#define SSM_SEL_DISPATCH_KPL(kpl, ...)                          \
    switch (kpl) {                                              \
        case 4: { constexpr int K_ = 4; __VA_ARGS__; } break;   \
        case 8: { constexpr int K_ = 8; __VA_ARGS__; } break;   \
        case 16: { constexpr int K_ = 16; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;                   \
    }
template <typename T, int NT, int VAR>
hipError_t sel_fwd_t(const SelFwdParams& p, int kpl, bool summary, hipStream_t st) {
    dim3 grid((p.D + 15) / 16, p.B, p.G), block(256);
    if (summary) { SSM_SEL_DISPATCH_KPL(kpl, sel_fwd_kernel<T, K_, NT, true, VAR><<<grid, block, 0, st>>>(p)) }
    else { SSM_SEL_DISPATCH_KPL(kpl, sel_fwd_kernel<T, K_, NT, false, VAR><<<grid, block, 0, st>>>(p)) }
    return hipGetLastError();
}
template <int VAR>
hipError_t launch_sel_fwd_var(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    const bool n16 = p.N == 16;
    if (dtype == 0)
        return n16 ? sel_fwd_t<float, 16, VAR>(p, kpl, summary, st) : sel_fwd_t<float, 0, VAR>(p, kpl, summary, st);
    return n16 ? sel_fwd_t<bf16_t, 16, VAR>(p, kpl, summary, st) : sel_fwd_t<bf16_t, 0, VAR>(p, kpl, summary, st);
}
template <typename T, int NT, int VAR>
hipError_t sel_bwd_t(const SelBwdParams& p, int kpl, bool summary, hipStream_t st) {
    dim3 grid((p.D + kBwdRows - 1) / kBwdRows, p.B, p.G), block(kBwdThreads);
    if (summary) { SSM_SEL_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, true, false, VAR><<<grid, block, 0, st>>>(p)) }
    else if (p.partA) { SSM_SEL_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, false, true, VAR><<<grid, block, 0, st>>>(p)) }
    else { SSM_SEL_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, false, false, VAR><<<grid, block, 0, st>>>(p)) }
    return hipGetLastError();
}
template <int VAR>
hipError_t launch_sel_bwd_var(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    const bool n16 = p.N == 16;
    if (dtype == 0)
        return n16 ? sel_bwd_t<float, 16, VAR>(p, kpl, summary, st) : sel_bwd_t<float, 0, VAR>(p, kpl, summary, st);
    return n16 ? sel_bwd_t<bf16_t, 16, VAR>(p, kpl, summary, st) : sel_bwd_t<bf16_t, 0, VAR>(p, kpl, summary, st);
}
#undef SSM_SEL_DISPATCH_KPL

}  // namespace ssm
