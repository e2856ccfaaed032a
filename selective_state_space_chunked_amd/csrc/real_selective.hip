// Diagonal real selective scan on gfx950: a_t[n] = exp(delta_t A[d,n]),
// b_t[n] = delta_t x_t B_t[n], y_t = sum_n C_t[n] h_t[n] (Mamba-style selection
// and discretisation, lpnh.cn "S3M" page, section 1.1; Euler input term).
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
// B_t and C_t are shared by all 16 rows and staged once per tile in LDS,
// transposed to [n][t] with 4 floats of padding after every lane's run so the
// 16-byte LDS reads of a row hit distinct banks.
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

// Stage a (TILE x N) block of a (B,L,N) tensor into LDS as float [n][t'].
// Steps beyond L read as zero.  NT = 16: one thread per step row, 16-byte loads.
template <typename T, int KPL, int NT, int THREADS = 256>
__device__ __forceinline__ void stage_tile(float* __restrict__ dst, const T* __restrict__ src, int b, int t0,
                                           int L, int N) {
    using G = TileGeom<KPL>;
    if constexpr (NT == 16) {
        for (int tt = threadIdx.x; tt < G::TILE; tt += THREADS) {
            const int t = t0 + tt;
            float v[16];
            if (t < L) load_run<16>(src + ((size_t)b * L + t) * 16, v, true);
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
            if (t < L) v = to_f32(src[((size_t)b * L + t) * N + n]);
            dst[G::idx(n, tt)] = v;
        }
    }
}

// Stage states [nb, ne) of a (TILE x N) block into rows 0 .. ne-nb-1 of dst.
// NT = 16 (halves of 8 states): one thread per step, 8 contiguous values.
template <typename T, int KPL, int NT, int NH, int THREADS = 256>
__device__ __forceinline__ void stage_states(float* __restrict__ dst, const T* __restrict__ src, int b, int t0,
                                             int L, int N, int nb, int ne) {
    using G = TileGeom<KPL>;
    if constexpr (NT == 16) {
        for (int tt = threadIdx.x; tt < G::TILE; tt += THREADS) {
            const int t = t0 + tt;
            float v[NH];
            if (t < L) load_run<NH>(src + ((size_t)b * L + t) * 16 + nb, v, true);
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
            if (t < L) v = to_f32(src[((size_t)b * L + t) * N + nb + n]);
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
// B and C tiles are staged eight states at a time (LDS 2 x 20.7 KB for KPL 16),
// so four workgroups fit on a CU next to the 128-VGPR budget of four waves per SIMD.
constexpr int kFwdStates = 8;

template <typename T, int KPL, int NT, bool SUMMARY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void sel_fwd_kernel(SelFwdParams p) {
    using G = TileGeom<KPL>;
    constexpr int TILE = G::TILE;
    constexpr int NH = kFwdStates;
    __shared__ __align__(16) float sB[NH * G::LDSW];
    __shared__ __align__(16) float sC[SUMMARY ? 4 : NH * G::LDSW];

    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;
    const T* __restrict__ delta = (const T*)p.delta;
    const T* __restrict__ xin = (const T*)p.x;
    const size_t seq = (size_t)b * p.D + dc;
    const size_t rowoff = seq * L;

    float A2 = 0.0f, carry = 0.0f, Pseg = 1.0f;
    if (lane < N) {
        A2 = p.A[(size_t)dc * N + lane] * kLog2e;
        if (!SUMMARY) {
            if (p.G > 1) carry = p.carry_in[(seq * p.G + g) * N + lane];
            else if (p.h0) carry = p.h0[seq * N + lane];
        }
    }
    const int tile0 = g * p.tiles_per_seg;
    const int tile1 = min(tile0 + p.tiles_per_seg, p.ntiles);
    const bool vec = p.vec != 0;

    for (int tile = tile0; tile < tile1; ++tile) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * KPL;
        const int nval = L - tl;
        float dl[KPL], dx[KPL];
        {
            float xv[KPL];
            load_steps<T, KPL>(delta + rowoff + tl, dl, nval, vec, p.stepf, dc);
            if (nval >= KPL) load_run<KPL>(xin + rowoff + tl, xv, vec);
            else load_run_masked<T, KPL>(xin + rowoff + tl, xv, nval);
#pragma unroll
            for (int j = 0; j < KPL; ++j) dx[j] = dl[j] * xv[j];
        }
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) dsum += dl[j];
        if (!SUMMARY && p.tile_dsum) {
            float ts = row_sum(dsum);
            if (act && lane == 0) p.tile_dsum[seq * p.ntiles + tile] = ts;
        }
        if (!SUMMARY && p.ckpt && act && lane < N) p.ckpt[(seq * p.ntiles + tile) * N + lane] = carry;

        float yacc[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) yacc[j] = 0.0f;

        for (int nb = 0; nb < N; nb += NH) {
            const int ne = min(nb + NH, N);
            __syncthreads();
            stage_states<T, KPL, NT, NH>(sB, (const T*)p.Bm, b, t0, L, N, nb, ne);
            if (!SUMMARY) stage_states<T, KPL, NT, NH>(sC, (const T*)p.C, b, t0, L, N, nb, ne);
            __syncthreads();
            // the broadcasts for state n+1 are issued while state n runs (lane n+1's
            // carry does not change during step n)
            float A2n_nx = row_bcast_rt(A2, nb), cin_nx = row_bcast_rt(carry, nb);
#pragma unroll 1
            for (int n = nb; n < ne; ++n) {
                const int nr = n - nb;   // row of state n in the staged half
                const float A2n = A2n_nx, cin = cin_nx;
                {
                    const int nn = min(n + 1, ne - 1);
                    A2n_nx = row_bcast_rt(A2, nn);
                    cin_nx = row_bcast_rt(carry, nn);
                }
                float bv[KPL], a[KPL], bx[KPL];
                read_run<KPL>(sB + nr * G::LDSW + lane * G::SEG, bv);
                float S = 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    a[j] = __builtin_amdgcn_exp2f(dl[j] * A2n);
                    bx[j] = dx[j] * bv[j];
                    S = fmaf(a[j], S, bx[j]);
                }
                float P = __builtin_amdgcn_exp2f(dsum * A2n);
                row_scan_affine_up(P, S);
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
                    read_run<KPL>(sC + nr * G::LDSW + lane * G::SEG, cv);
#pragma unroll
                    for (int j = 0; j < KPL; ++j) {
                        h = fmaf(a[j], h, bx[j]);
                        yacc[j] = fmaf(cv[j], h, yacc[j]);
                    }
                }
                carry = (lane == n) ? newc : carry;
            }
        }
        if (!SUMMARY && p.y && act && nval > 0)
            store_run<KPL>((T*)p.y + rowoff + tl, yacc, vec, nval);
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
// ---------------------------------------------------------------------------
template <typename T, int KPL, int NT, bool SUMMARY, bool WA>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void sel_bwd_kernel(SelBwdParams p) {
    using G = TileGeom<KPL>;
    constexpr int TILE = G::TILE;
    constexpr int ROWS = kBwdRows;
    __shared__ __align__(16) float sB[SUMMARY ? 4 : 16 * G::LDSW];
    __shared__ __align__(16) float sC[16 * G::LDSW];
    // Partials of gB and gC for one state after the in-wave pre-sum, laid out
    // like the B/C tiles ([pre-summed row][lane run + 4 pad]); two buffers
    // (state parity) so one barrier per state suffices.
    constexpr int RB = ROWS / kPresum;
    __shared__ __align__(16) float red[SUMMARY ? 4 : 2 * 2 * RB * G::LDSW];

    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * ROWS + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;
    const T* __restrict__ delta = (const T*)p.delta;
    const T* __restrict__ xin = (const T*)p.x;
    const T* __restrict__ gyin = (const T*)p.gy;
    const size_t seq = (size_t)b * p.D + dc;
    const size_t rowoff = seq * L;
    const bool vec = p.vec != 0;
    const bool wantB = p.partB != nullptr, wantC = p.partC != nullptr;

    float A2 = 0.0f, nu = 0.0f, gAacc = 0.0f, Qseg = 1.0f, gbias = 0.0f;
    if (lane < N) {
        A2 = p.A[(size_t)dc * N + lane] * kLog2e;
        if (!SUMMARY) {
            if (p.G > 1) nu = p.nu_in[(seq * p.G + g) * N + lane];
            else if (p.gh_last) nu = p.gh_last[seq * N + lane];
        }
    }
    const int tile0 = g * p.tiles_per_seg;
    const int tile1 = min(tile0 + p.tiles_per_seg, p.ntiles);

    for (int tile = tile1 - 1; tile >= tile0; --tile) {
        const int t0 = tile * TILE;
        __syncthreads();
        if (!SUMMARY) stage_tile<T, KPL, NT, kBwdThreads>(sB, (const T*)p.Bm, b, t0, L, N);
        stage_tile<T, KPL, NT, kBwdThreads>(sC, (const T*)p.C, b, t0, L, N);
        __syncthreads();

        const int tl = t0 + lane * KPL;
        const int nval = L - tl;
        float dl[KPL], dx[KPL], gyv[KPL];
        {
            float xv[KPL];
            load_steps<T, KPL>(delta + rowoff + tl, dl, nval, vec, p.stepf, dc);
            if (nval >= KPL) {
                load_run<KPL>(gyin + rowoff + tl, gyv, vec);
                if (!SUMMARY) load_run<KPL>(xin + rowoff + tl, xv, vec);
            } else {
                load_run_masked<T, KPL>(gyin + rowoff + tl, gyv, nval);
                if (!SUMMARY) load_run_masked<T, KPL>(xin + rowoff + tl, xv, nval);
            }
            // rows past D contribute nothing to the sums over channels
            const float live = act ? 1.0f : 0.0f;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                dx[j] = SUMMARY ? 0.0f : dl[j] * xv[j] * live;
                if (!SUMMARY) gyv[j] *= live;
            }
        }
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) dsum += dl[j];
        float hs = 0.0f;
        if (!SUMMARY && lane < N) hs = p.ckpt[(seq * p.ntiles + tile) * N + lane];

        float Gd[KPL], Sb[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) { Gd[j] = 0.0f; Sb[j] = 0.0f; }

        // broadcasts of state n+1 are issued while state n runs (lane n+1's adjoint
        // does not change during step n)
        float A2n_nx = row_bcast_rt(A2, 0), nin_nx = row_bcast_rt(nu, 0), cin_nx = row_bcast_rt(hs, 0);
        const int n_end = NT ? NT : N;
#pragma unroll 1
        for (int n = 0; n < n_end; ++n) {
            const float A2n = A2n_nx, nin = nin_nx, cin = cin_nx;
            {
                const int nn = min(n + 1, n_end - 1);
                A2n_nx = row_bcast_rt(A2, nn);
                nin_nx = row_bcast_rt(nu, nn);
                if (!SUMMARY) cin_nx = row_bcast_rt(hs, nn);
            }
            float a[KPL], cv[KPL];
            read_run<KPL>(sC + n * G::LDSW + lane * G::SEG, cv);
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
                float bv[KPL], bx[KPL], h[KPL + 1];
                read_run<KPL>(sB + n * G::LDSW + lane * G::SEG, bv);
                float S = 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    bx[j] = dx[j] * bv[j];
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
                    Sb[j] = fmaf(lam, bv[j], Sb[j]);
                    if constexpr (WA) gAl = fmaf(t1, dl[j], gAl);
                    pB[j] = lam * dx[j];
                    pC[j] = gyv[j] * h[j + 1];
                }
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
                    if constexpr (CNT % 4 == 0) {
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
                    __syncthreads();
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
        if (!SUMMARY && act && nval > 0) {
            if (p.gx) {
                float v[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) v[j] = dl[j] * Sb[j];
                store_run<KPL>((T*)p.gx + rowoff + tl, v, vec, nval);
            }
            if (p.gdelta || p.partBias) {
                // gradient w.r.t. delta as given (the projection output when the
                // step sizes are transformed): d delta/d z times d Loss/d delta
                float xv[KPL], v[KPL];
                if (nval >= KPL) load_run<KPL>(xin + rowoff + tl, xv, vec);
                else load_run_masked<T, KPL>(xin + rowoff + tl, xv, nval);
#pragma unroll
                for (int j = 0; j < KPL; ++j)
                    v[j] = fmaf(xv[j], Sb[j], Gd[j]) * step_xform_grad(dl[j], p.stepf.softplus);
                if (p.gdelta) store_run<KPL>((T*)p.gdelta + rowoff + tl, v, vec, nval);
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

// ---------------------------------------------------------------------------
// segment combines (phase B across segments), one lane per (sequence, state)
// ---------------------------------------------------------------------------
__global__ void seg_combine_fwd_kernel(const float* __restrict__ P, const float* __restrict__ S,
                                       const float* __restrict__ h0, float* __restrict__ carry_in, int BD,
                                       int G, int N) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BD * N) return;
    const int s = i / N, n = i - s * N;
    float h = h0 ? h0[(size_t)s * N + n] : 0.0f;
    for (int g = 0; g < G; ++g) {
        const size_t o = ((size_t)s * G + g) * N + n;
        carry_in[o] = h;
        h = fmaf(P[o], h, S[o]);
    }
}
__global__ void seg_combine_rev_kernel(const float* __restrict__ Q, const float* __restrict__ R,
                                       const float* __restrict__ nu_last, float* __restrict__ nu_in, int BD,
                                       int G, int N) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BD * N) return;
    const int s = i / N, n = i - s * N;
    float v = nu_last ? nu_last[(size_t)s * N + n] : 0.0f;
    for (int g = G - 1; g >= 0; --g) {
        const size_t o = ((size_t)s * G + g) * N + n;
        nu_in[o] = v;
        v = fmaf(Q[o], v, R[o]);
    }
}

// partial (nblk,B,N,L) -> out (B,L,N), adding the blocks in index order
// Channel-block partials (nblk, B, N, L) of gB and gC -> outputs (B, L, N).
// A workgroup takes 64 steps of one batch row and one tensor (blockIdx.z);
// thread (n, q) adds the nblk partials of steps 4q..4q+3 in block order, then
// the 64 x N tile is transposed through LDS so the (t, n) output rows are
// written contiguously.
template <typename T>
__global__ __launch_bounds__(256) void reduce_parts_btn_kernel(const float* __restrict__ partB,
                                                               const float* __restrict__ partC, int nblk, int B,
                                                               int N, int L, T* __restrict__ outB,
                                                               T* __restrict__ outC) {
    __shared__ float tile[64][17];
    const float* __restrict__ part = blockIdx.z ? partC : partB;
    T* __restrict__ out = blockIdx.z ? outC : outB;
    if (!part || !out) return;
    const int b = blockIdx.y, t0 = blockIdx.x * 64;
    const int n = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int tl = 4 * q, t = t0 + tl;
    const size_t stride = (size_t)B * N * L;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (n < N) {
        const float* src = part + ((size_t)b * N + n) * L + t;
        if ((L & 3) == 0 && t < L) {
            // sixteen loads in flight per thread; the additions stay in block order
            int k = 0;
            for (; k + 16 <= nblk; k += 16) {
                float4 v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const float4*>(src + (size_t)(k + u) * stride);
#pragma unroll
                for (int u = 0; u < 16; ++u) { s[0] += v[u].x; s[1] += v[u].y; s[2] += v[u].z; s[3] += v[u].w; }
            }
            for (; k < nblk; ++k) {
                const float4 v = *reinterpret_cast<const float4*>(src + (size_t)k * stride);
                s[0] += v.x; s[1] += v.y; s[2] += v.z; s[3] += v.w;
            }
        } else {
            for (int k = 0; k < nblk; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (t + i < L) s[i] += src[(size_t)k * stride + i];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[tl + i][n] = s[i];
    __syncthreads();
    const int steps = min(64, L - t0);
    T* dst = out + ((size_t)b * L + t0) * N;
    for (int i = threadIdx.x; i < steps * N; i += 256) dst[i] = from_f32<T>(tile[i / N][i % N]);
}
// The same sums when N and L are multiples of 4: wave w of the workgroup takes
// state n = 4 * blockIdx.z' + w and lane l the steps t0 + 4l .. t0 + 4l + 3, so
// every load instruction reads 1 KB of one partial row contiguously; each
// thread then stores the four states of one step.  Additions in block order,
// as above (the two kernels give identical sums).
template <typename T>
__global__ __launch_bounds__(256) void reduce_parts_btn4_kernel(const float* __restrict__ partB,
                                                                const float* __restrict__ partC, int nblk, int B,
                                                                int N, int L, T* __restrict__ outB,
                                                                T* __restrict__ outC) {
    __shared__ float tile[256][5];
    const int nq = N >> 2;
    const int which = blockIdx.z / nq, n0 = 4 * (blockIdx.z - which * nq);
    const float* __restrict__ part = which ? partC : partB;
    T* __restrict__ out = which ? outC : outB;
    if (!part || !out) return;
    const int b = blockIdx.y, t0 = blockIdx.x * 256;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int t = t0 + 4 * l;
    const size_t stride = (size_t)B * N * L;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t < L) {
        const float* src = part + ((size_t)b * N + n0 + w) * L + t;
        int k = 0;
        for (; k + 16 <= nblk; k += 16) {
            float4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = *reinterpret_cast<const float4*>(src + (size_t)(k + u) * stride);
#pragma unroll
            for (int u = 0; u < 16; ++u) { s[0] += v[u].x; s[1] += v[u].y; s[2] += v[u].z; s[3] += v[u].w; }
        }
        for (; k < nblk; ++k) {
            const float4 v = *reinterpret_cast<const float4*>(src + (size_t)k * stride);
            s[0] += v.x; s[1] += v.y; s[2] += v.z; s[3] += v.w;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[4 * l + i][w] = s[i];
    __syncthreads();
    const int tt = t0 + threadIdx.x;
    if (tt < L) {
        T* dst = out + ((size_t)b * L + tt) * N + n0;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(tile[threadIdx.x][i]);
    }
}
// partial (B,G,D,N) -> out (D,N)
__global__ void reduce_parts_dn_kernel(const float* __restrict__ part, int B, int G, int D, int N,
                                       float* __restrict__ out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= D * N) return;
    float s = 0.0f;
    for (int k = 0; k < B * G; ++k) s += part[(size_t)k * D * N + i];
    out[i] = s;
}

// ---------------------------------------------------------------------------
// impulse sensitivity: s_t = delta_t sum_n B_t[n] C_out[n] exp2(A2[n] S_t),
// S_t = sum_{s=t+1..t_out} delta_s (the reverse costate mu_t = C_out prod a in
// closed form).  The suffix sums over tiles come from a per-sequence pass in
// double precision; inside a tile they are DPP row suffix sums plus in-lane
// suffix sums.  Every tile is independent, so the grid spans all tiles.
// ---------------------------------------------------------------------------
template <typename T, int KPL>
__global__ void tile_dsum_kernel(const T* __restrict__ delta, StepXform stepf, float* __restrict__ out, int B,
                                 int D, int L, int ntiles) {
    const int lane = threadIdx.x & 15, row = threadIdx.x >> 4;
    const int d = blockIdx.x * 16 + row, b = blockIdx.y;
    const bool act = d < D;
    const int dc = act ? d : D - 1;
    for (int tile = blockIdx.z; tile < ntiles; tile += gridDim.z) {   // grid.z is capped at 65535
        const int tl = tile * 16 * KPL + lane * KPL;
        float v[KPL];
        load_steps<T, KPL>(delta + ((size_t)b * D + dc) * L + tl, v, L - tl, false, stepf, dc);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) s += v[j];
        s = row_sum(s);
        if (act && lane == 0) out[((size_t)b * D + dc) * ntiles + tile] = s;
    }
}

// send[s, k] = sum of delta over the steps of tiles after k, up to t_out, in
// double.  One workgroup per sequence: tile contributions (whole tile sums
// before t_out's tile, the partial sum of t_out's tile, zero after it) are
// taken in blocks of 256 from the end, suffix-scanned in LDS, and each
// block's total is carried to the next.
template <typename T>
__global__ __launch_bounds__(256) void sens_suffix_kernel(const T* __restrict__ delta, StepXform stepf,
                                                          const float* __restrict__ tile_dsum,
                                                          double* __restrict__ send, int D, int L, int ntiles,
                                                          int tile_len, int t_out) {
    __shared__ double sc[257];
    const int s = blockIdx.x, tid = threadIdx.x;
    const int tout_tile = t_out / tile_len;
    // partial sum of t_out's own tile (fixed-order tree reduction)
    double part = 0.0;
    const float bias = stepf.bias ? stepf.bias[s % D] : 0.0f;
    const bool xf = stepf.bias != nullptr || stepf.softplus;
    for (int t = tout_tile * tile_len + tid; t <= t_out; t += 256) {
        const float z = to_f32(delta[(size_t)s * L + t]);
        part += (double)(xf ? step_xform(z, bias, stepf.softplus) : z);
    }
    sc[tid] = part;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) sc[tid] += sc[tid + w];
        __syncthreads();
    }
    const double tpart = sc[0];
    __syncthreads();
    double carry = 0.0;
    for (int base = ((ntiles - 1) / 256) * 256; base >= 0; base -= 256) {
        const int k = base + tid;
        double c = 0.0;
        if (k < tout_tile) c = (double)tile_dsum[(size_t)s * ntiles + k];
        else if (k == tout_tile) c = tpart;
        sc[tid] = c;
        if (tid == 0) sc[256] = 0.0;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {   // inclusive suffix scan
            const double v = tid + off < 256 ? sc[tid + off] : 0.0;
            __syncthreads();
            sc[tid] += v;
            __syncthreads();
        }
        if (k < ntiles) send[(size_t)s * ntiles + k] = carry + sc[tid + 1];   // tiles after k
        const double tot = sc[0];
        __syncthreads();
        carry += tot;
    }
}

// Tiles per sensitivity workgroup: the next tile's B values and step sizes
// are loaded while the current tile is computed.
constexpr int kSensTiles = 4;

// WD: also s_delta_t = d y[t_out] / d delta_t = sum_n mu_t[n] (A[n] a_t[n] h_{t-1}[n] + x_t B_t[n])
//     = x_t * (the s_x sum) + sum_n C_out[n] A[n] 2^(A2[n] (S_t + delta_t)) h_{t-1}[n],
// with the states h re-run inside the tile from its checkpoint (lane fold, DPP
// scan, re-run, as in the forward).  B is then staged without the C_out factor.
template <typename T, int KPL, int NT, bool WD = false>
__global__ __launch_bounds__(256) void sens_kernel(SensParams p) {
    using Gm = TileGeom<KPL>;
    constexpr int TILE = Gm::TILE;
    constexpr int SPT = NT ? TILE * NT / 256 : 1;   // staged values per thread (N = 16)
    __shared__ __align__(16) float sBC[16 * Gm::LDSW];
    __shared__ float sCout[16];
    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;
    const size_t seq = (size_t)b * p.D + dc;
    const int tile0 = blockIdx.z * p.tiles_per_wg;
    const int tile1 = min(tile0 + p.tiles_per_wg, p.ntiles);
    const T* Bm = (const T*)p.Bm;
    const bool vec = p.vec != 0;
    if (tid < N) sCout[tid] = to_f32(((const T*)p.C)[((size_t)b * L + p.t_out) * N + tid]);
    float A2 = 0.0f;
    if (lane < N) A2 = p.A[(size_t)dc * N + lane] * kLog2e;
    // B of one tile: thread tid holds entries e = tid + 256 i, e = tt * N + n
    auto fetchB = [&](int tile, float (&v)[SPT]) {
        const int t0 = tile * TILE;
        if constexpr (NT != 0) {
#pragma unroll
            for (int q = 0; q < SPT; ++q) {
                const int e = tid + 256 * q, tt = e / NT;
                v[q] = t0 + tt < L ? to_f32(Bm[((size_t)b * L + t0) * NT + e]) : 0.0f;
            }
        }
    };
    auto putB = [&](int tile, const float (&v)[SPT]) {
        if constexpr (NT != 0) {
#pragma unroll
            for (int q = 0; q < SPT; ++q) {
                const int e = tid + 256 * q, tt = e / NT, n = e - tt * NT;
                sBC[Gm::idx(n, tt)] = WD ? v[q] : v[q] * sCout[n];
            }
        } else {
            const int t0 = tile * TILE;
            for (int e = tid; e < TILE * N; e += 256) {
                const int tt = e / N, n = e - tt * N;
                const int t = t0 + tt;
                sBC[Gm::idx(n, tt)] = t < L ? to_f32(Bm[((size_t)b * L + t) * N + n]) * (WD ? 1.0f : sCout[n]) : 0.0f;
            }
        }
    };
    float nb[SPT];
    fetchB(tile0, nb);
    __syncthreads();          // sCout
    putB(tile0, nb);
    __syncthreads();
    for (int tile = tile0; tile < tile1; ++tile) {
        const int t0 = tile * TILE;
        const int tl = t0 + lane * KPL;
        if (t0 > p.t_out) {   // tile after t_out: zero sensitivity (uniform: later tiles are too)
            if (act && tl < L) {
                float z[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) z[j] = 0.0f;
                if (p.s) store_run<KPL>((T*)p.s + seq * L + tl, z, vec, L - tl);
                if (WD) store_run<KPL>((T*)p.s_delta + seq * L + tl, z, vec, L - tl);
            }
            continue;
        }
        const bool more = tile + 1 < tile1 && (tile + 1) * TILE <= p.t_out;
        if (more) fetchB(tile + 1, nb);   // in flight while this tile runs
        float dl[KPL];
        load_steps<T, KPL>((const T*)p.delta + seq * L + tl, dl, min(L, p.t_out + 1) - tl, false, p.stepf, dc);
        // S_j = sum of delta over steps after j up to t_out
        float lsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) lsum += dl[j];
        const float base = (float)p.send[seq * p.ntiles + tile] + row_excl_sum_down(lsum);
        float S[KPL];
        {
            float run = 0.0f;
#pragma unroll
            for (int j = KPL - 1; j >= 0; --j) {
                S[j] = base + run;
                run += dl[j];
            }
        }
        float acc[KPL], gd[KPL], xv[KPL], hin = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) { acc[j] = 0.0f; gd[j] = 0.0f; }
        if (WD) {
            load_run_masked<T, KPL>((const T*)p.x + seq * L + tl, xv, min(L, p.t_out + 1) - tl);
            if (lane < N) hin = p.ckpt[(seq * p.ntiles + tile) * N + lane];   // state entering the tile
        }
        for_states<NT>(N, [&](auto st) {
            const float A2n = st.bc(A2);
            float bc[KPL], e[KPL];
            read_run<KPL>(sBC + st.n * Gm::LDSW + lane * Gm::SEG, bc);
#pragma unroll
            for (int j = 0; j < KPL; ++j) e[j] = __builtin_amdgcn_exp2f(A2n * S[j]);
            if constexpr (!WD) {
#pragma unroll
                for (int j = 0; j < KPL; ++j) acc[j] = fmaf(bc[j], e[j], acc[j]);
            } else {
                const float Cn = sCout[st.n];
                float a[KPL], bx[KPL], Sf = 0.0f;
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    acc[j] = fmaf(bc[j] * Cn, e[j], acc[j]);
                    a[j] = __builtin_amdgcn_exp2f(dl[j] * A2n);
                    bx[j] = dl[j] * xv[j] * bc[j];
                    Sf = fmaf(a[j], Sf, bx[j]);
                }
                float Pf = __builtin_amdgcn_exp2f(lsum * A2n);
                row_scan_affine_up(Pf, Sf);
                const float cin = st.bc(hin);
                float h = dpp<SSM_DPP_ROW_SHR(1)>(cin, fmaf(Pf, cin, Sf));   // state entering this lane's run
                const float CA = Cn * (A2n * kLn2);
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    gd[j] = fmaf(CA, e[j] * a[j] * h, gd[j]);
                    h = fmaf(a[j], h, bx[j]);
                }
            }
        });
        if (act && tl < L) {
            float v[KPL];
            if (p.s) {
#pragma unroll
                for (int j = 0; j < KPL; ++j) v[j] = (tl + j <= p.t_out) ? dl[j] * acc[j] : 0.0f;
                store_run<KPL>((T*)p.s + seq * L + tl, v, vec, L - tl);
            }
            if (WD) {
#pragma unroll
                for (int j = 0; j < KPL; ++j)
                    v[j] = (tl + j <= p.t_out)
                               ? fmaf(xv[j], acc[j], gd[j]) * step_xform_grad(dl[j], p.stepf.softplus)
                               : 0.0f;
                store_run<KPL>((T*)p.s_delta + seq * L + tl, v, vec, L - tl);
            }
        }
        if (more) {
            __syncthreads();   // every lane is done with this tile's values
            putB(tile + 1, nb);
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Rows of the input Jacobian (PGF page, abstract: sensitivities of the outputs
// to the inputs by reverse evolution of the costate).  For the output steps
// tau_r = t0 + r, r < R:
//   s[r, t] = delta_t sum_n B_t[n] C_{tau_r}[n] prod_{t < u <= tau_r} a_u[n]    (t <= tau_r), 0 after.
// For t <= t0 the product splits at t0: prod_{t < u <= t0} a_u[n] = 2^(A2[n] S_t)
// with S_t the sum of delta over (t, t0] (the costate of row t0), and
//   w_r[n] = C_{tau_r}[n] prod_{t0 < u <= tau_r} a_u[n],
// so s[r, t] = delta_t sum_n (B_t[n] 2^(A2[n] S_t)) w_r[n]: one exp per (t, n)
// for all R rows.  Both factors are products of a's, as in the direct form.
// The few steps t in (t0, t0 + R) use the direct form in a second kernel.
// Output layout (R, B, D, L): row r is a (B, D, L) slab; every store of a
// 16-lane row covers 64 consecutive steps of one row.
// ---------------------------------------------------------------------------

// One thread per (sequence, row r).  D_k = sum of delta over (t0, t0 + k].
// TAIL = false: w_r into the workspace (before the main pass); TAIL = true:
// the entries s[r, t] for t in (t0, t0 + R) by the direct form (after it).
template <typename T, bool TAIL>
__global__ __launch_bounds__(256) void sens_rows_edge_kernel(SensRowsParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.D * p.R) return;
    const int R = p.R, r = i % R, sq = i / R, d = sq % p.D, b = sq / p.D;
    const int N = p.N, L = p.L, t0 = p.t0, tau = t0 + r;
    const T* delta = (const T*)p.delta + (size_t)sq * L;
    const T* Bm = (const T*)p.Bm + (size_t)b * L * N;
    const T* C = (const T*)p.C + (size_t)b * L * N;
    const float* A = p.A + (size_t)d * N;
    const float bias = p.stepf.bias ? p.stepf.bias[d] : 0.0f;
    auto step = [&](int t) { return step_xform(to_f32(delta[t]), bias, p.stepf.softplus); };
    float Dr = 0.0f;
    for (int k = 1; k <= r; ++k) Dr += step(t0 + k);
    if (!TAIL) {
        float* w = p.w + ((size_t)sq * R + r) * N;
        for (int n = 0; n < N; ++n) w[n] = to_f32(C[(size_t)tau * N + n]) * __builtin_amdgcn_exp2f(A[n] * kLog2e * Dr);
        return;
    }
    T* out = (T*)p.s + ((size_t)r * p.B * p.D + sq) * L;
    float Dk = 0.0f;
    for (int k = 1; k < R; ++k) {
        const int t = t0 + k;
        float v = 0.0f;
        if (k <= r) {
            const float dt = step(t);
            Dk += dt;
            for (int n = 0; n < N; ++n)
                v = fmaf(to_f32(Bm[(size_t)t * N + n]) * to_f32(C[(size_t)tau * N + n]),
                         __builtin_amdgcn_exp2f(A[n] * kLog2e * (Dr - Dk)), v);
            v *= dt;
        }
        out[t] = from_f32<T>(v);
    }
}

// Main pass: 64-step tiles, 16 sequences per workgroup, lane l owns 4 steps;
// per state n one exp per step and kSensRowsMax multiply-adds against the row
// weights (zero past R).  Every step gets a value: step sizes past t0 load as
// 0, so steps t > t0 come out 0, and the tail kernel then overwrites
// (t0, t0 + R).
template <typename T, int NT>
__global__ __launch_bounds__(256) void sens_rows_kernel(SensRowsParams p) {
    constexpr int KPL = 4, RM = kSensRowsMax;
    using Gm = TileGeom<KPL>;
    constexpr int TILE = Gm::TILE;
    __shared__ __align__(16) float sB[16 * Gm::LDSW];
    __shared__ __align__(16) float sW[16 * 16 * RM];    // [row][n][r]
    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L, R = p.R, t0 = p.t0;
    const size_t seq = (size_t)b * p.D + dc;
    const size_t plane = (size_t)p.B * p.D * L;   // elements per output row
    const bool vec = p.vec != 0;
    for (int e = tid; e < 16 * 16 * RM; e += 256) {
        const int rw = e / (16 * RM), n = (e / RM) % 16, r = e % RM;
        const int dd = min(blockIdx.x * 16 + rw, p.D - 1);
        sW[e] = (n < N && r < R) ? p.w[(((size_t)b * p.D + dd) * R + r) * N + n] : 0.0f;
    }
    float A2 = 0.0f;
    if (lane < N) A2 = p.A[(size_t)dc * N + lane] * kLog2e;
    const int tile0 = blockIdx.z * p.tiles_per_wg;
    const int tile1 = min(tile0 + p.tiles_per_wg, p.ntiles);
    for (int tile = tile0; tile < tile1; ++tile) {
        const int ts = tile * TILE;
        const int tl = ts + lane * KPL;
        T* o = (T*)p.s + seq * L + tl;   // this lane's first step in row 0
        if (ts > t0) {   // tiles after t0 (uniform; later tiles too): zeros
            if (act && tl < L) {
                const float z[KPL] = {};
                for (int r = 0; r < R; ++r) store_run<KPL>(o + r * plane, z, vec, L - tl);
            }
            continue;
        }
        __syncthreads();   // sW ready (first tile) / the previous tile's B no longer read
        if constexpr (NT == 16) {
            const int tt = tid >> 2, q = tid & 3;   // 64 steps x 4 quarters of 4 states
            const int t = ts + tt;
            float v[4];
            if (t < L) load_run<4>((const T*)p.Bm + ((size_t)b * L + t) * 16 + 4 * q, v, true);
            else v[0] = v[1] = v[2] = v[3] = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) sB[Gm::idx(4 * q + k, tt)] = v[k];
        } else {
            for (int e = tid; e < TILE * N; e += 256) {
                const int tt = e / N, n = e - tt * N, t = ts + tt;
                sB[Gm::idx(n, tt)] = t < L ? to_f32(((const T*)p.Bm)[((size_t)b * L + t) * N + n]) : 0.0f;
            }
        }
        __syncthreads();
        float dl[KPL];
        load_steps<T, KPL>((const T*)p.delta + seq * L + tl, dl, min(L, t0 + 1) - tl, false, p.stepf, dc);
        // S_j = sum of delta over steps after j up to t0
        float lsum = 0.0f;
#pragma unroll
        for (int j = 0; j < KPL; ++j) lsum += dl[j];
        const float base = (float)p.send[seq * p.ntiles + tile] + row_excl_sum_down(lsum);
        float S[KPL];
        {
            float run = 0.0f;
#pragma unroll
            for (int j = KPL - 1; j >= 0; --j) {
                S[j] = base + run;
                run += dl[j];
            }
        }
        float acc[RM][KPL];
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
            for (int j = 0; j < KPL; ++j) acc[r][j] = 0.0f;
        auto body = [&](auto st) {
            const float A2n = st.bc(A2);
            float m[KPL];
            read_run<KPL>(sB + st.n * Gm::LDSW + lane * Gm::SEG, m);
#pragma unroll
            for (int j = 0; j < KPL; ++j) m[j] *= __builtin_amdgcn_exp2f(A2n * S[j]);
            float wv[RM];
            read_run<RM>(sW + (row * 16 + st.n) * RM, wv);
#pragma unroll
            for (int r = 0; r < RM; ++r)
#pragma unroll
                for (int j = 0; j < KPL; ++j) acc[r][j] = fmaf(m[j], wv[r], acc[r][j]);
        };
        for_states<NT>(N, body);
        if (act && tl < L) {
#pragma unroll
            for (int r = 0; r < RM; ++r)   // predicated, not exited: acc stays in registers
                if (r < R) {
                    float v[KPL];
#pragma unroll
                    for (int j = 0; j < KPL; ++j) v[j] = dl[j] * acc[r][j];
                    store_run<KPL>(o + r * plane, v, vec, L - tl);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define SSM_DISPATCH_KPL(kpl, ...)                         \
    switch (kpl) {                                         \
        case 4: { constexpr int K_ = 4; __VA_ARGS__; } break;   \
        case 8: { constexpr int K_ = 8; __VA_ARGS__; } break;   \
        case 16: { constexpr int K_ = 16; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;              \
    }

template <typename T, int NT>
hipError_t sel_fwd_t(const SelFwdParams& p, int kpl, bool summary, hipStream_t st) {
    dim3 grid((p.D + 15) / 16, p.B, p.G), block(256);
    if (summary) { SSM_DISPATCH_KPL(kpl, sel_fwd_kernel<T, K_, NT, true><<<grid, block, 0, st>>>(p)) }
    else { SSM_DISPATCH_KPL(kpl, sel_fwd_kernel<T, K_, NT, false><<<grid, block, 0, st>>>(p)) }
    return hipGetLastError();
}
hipError_t launch_sel_fwd(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    const bool n16 = p.N == 16;
    if (dtype == 0) return n16 ? sel_fwd_t<float, 16>(p, kpl, summary, st) : sel_fwd_t<float, 0>(p, kpl, summary, st);
    return n16 ? sel_fwd_t<bf16_t, 16>(p, kpl, summary, st) : sel_fwd_t<bf16_t, 0>(p, kpl, summary, st);
}

template <typename T, int NT>
hipError_t sel_bwd_t(const SelBwdParams& p, int kpl, bool summary, hipStream_t st) {
    dim3 grid((p.D + kBwdRows - 1) / kBwdRows, p.B, p.G), block(kBwdThreads);
    if (summary) { SSM_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, true, false><<<grid, block, 0, st>>>(p)) }
    else if (p.partA) { SSM_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, false, true><<<grid, block, 0, st>>>(p)) }
    else { SSM_DISPATCH_KPL(kpl, sel_bwd_kernel<T, K_, NT, false, false><<<grid, block, 0, st>>>(p)) }
    return hipGetLastError();
}
int sel_bwd_rows() { return kBwdRows; }
hipError_t launch_sel_bwd(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st) {
    const bool n16 = p.N == 16;
    if (dtype == 0) return n16 ? sel_bwd_t<float, 16>(p, kpl, summary, st) : sel_bwd_t<float, 0>(p, kpl, summary, st);
    return n16 ? sel_bwd_t<bf16_t, 16>(p, kpl, summary, st) : sel_bwd_t<bf16_t, 0>(p, kpl, summary, st);
}

hipError_t launch_seg_combine_fwd(const float* P, const float* S, const float* h0, float* carry_in, int BD,
                                  int G, int N, hipStream_t st) {
    const int total = BD * N;
    seg_combine_fwd_kernel<<<(total + 255) / 256, 256, 0, st>>>(P, S, h0, carry_in, BD, G, N);
    return hipGetLastError();
}
hipError_t launch_seg_combine_rev(const float* Q, const float* R, const float* nu_last, float* nu_in, int BD,
                                  int G, int N, hipStream_t st) {
    const int total = BD * N;
    seg_combine_rev_kernel<<<(total + 255) / 256, 256, 0, st>>>(Q, R, nu_last, nu_in, BD, G, N);
    return hipGetLastError();
}
hipError_t launch_reduce_parts_btn(const float* partB, const float* partC, int nblk, int B, int N, int L,
                                   void* outB, void* outC, int dtype, hipStream_t st) {
    if (N % 4 == 0 && L % 4 == 0) {
        dim3 g4((unsigned)((L + 255) / 256), (unsigned)B, (unsigned)(2 * (N / 4)));
        if (dtype == 0)
            reduce_parts_btn4_kernel<float><<<g4, 256, 0, st>>>(partB, partC, nblk, B, N, L, (float*)outB,
                                                                (float*)outC);
        else
            reduce_parts_btn4_kernel<bf16_t><<<g4, 256, 0, st>>>(partB, partC, nblk, B, N, L, (bf16_t*)outB,
                                                                 (bf16_t*)outC);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((L + 63) / 64), (unsigned)B, 2);
    if (dtype == 0)
        reduce_parts_btn_kernel<float><<<grid, 256, 0, st>>>(partB, partC, nblk, B, N, L, (float*)outB, (float*)outC);
    else
        reduce_parts_btn_kernel<bf16_t><<<grid, 256, 0, st>>>(partB, partC, nblk, B, N, L, (bf16_t*)outB,
                                                              (bf16_t*)outC);
    return hipGetLastError();
}
hipError_t launch_reduce_parts_dn(const float* part, int B, int G, int D, int N, float* out, hipStream_t st) {
    reduce_parts_dn_kernel<<<(D * N + 255) / 256, 256, 0, st>>>(part, B, G, D, N, out);
    return hipGetLastError();
}
hipError_t launch_tile_dsum(const void* delta, StepXform stepf, float* tile_dsum, int B, int D, int L, int ntiles,
                            int kpl, int dtype, hipStream_t st) {
    dim3 grid((D + 15) / 16, B, std::min(ntiles, 65535));
    if (dtype == 0) {
        SSM_DISPATCH_KPL(kpl, tile_dsum_kernel<float, K_><<<grid, 256, 0, st>>>((const float*)delta, stepf, tile_dsum,
                                                                                  B, D, L, ntiles))
    } else {
        SSM_DISPATCH_KPL(kpl, tile_dsum_kernel<bf16_t, K_><<<grid, 256, 0, st>>>((const bf16_t*)delta, stepf,
                                                                                   tile_dsum, B, D, L, ntiles))
    }
    return hipGetLastError();
}
hipError_t launch_sens_suffix(const void* delta, StepXform stepf, const float* tile_dsum, double* send, int B, int D,
                              int L, int ntiles, int tile_len, int t_out, int dtype, hipStream_t st) {
    const int BD = B * D;
    if (dtype == 0)
        sens_suffix_kernel<float><<<BD, 256, 0, st>>>((const float*)delta, stepf, tile_dsum, send, D, L, ntiles,
                                                      tile_len, t_out);
    else
        sens_suffix_kernel<bf16_t><<<BD, 256, 0, st>>>((const bf16_t*)delta, stepf, tile_dsum, send, D, L, ntiles,
                                                       tile_len, t_out);
    return hipGetLastError();
}
// Tiles per workgroup: kSensTiles, more when the sequence has so many tiles
// that grid.z would pass its 65535 limit.
static int sens_tiles_per_wg(int ntiles) { return std::max(kSensTiles, (ntiles + 65534) / 65535); }

hipError_t launch_sens(const SensParams& pin, int dtype, int kpl, hipStream_t st) {
    SensParams p = pin;
    p.tiles_per_wg = sens_tiles_per_wg(p.ntiles);
    dim3 grid((p.D + 15) / 16, p.B, (p.ntiles + p.tiles_per_wg - 1) / p.tiles_per_wg);
    const bool n16 = p.N == 16;
    if (p.s_delta) {
        if (dtype == 0) {
            if (n16) { SSM_DISPATCH_KPL(kpl, sens_kernel<float, K_, 16, true><<<grid, 256, 0, st>>>(p)) }
            else { SSM_DISPATCH_KPL(kpl, sens_kernel<float, K_, 0, true><<<grid, 256, 0, st>>>(p)) }
        } else {
            if (n16) { SSM_DISPATCH_KPL(kpl, sens_kernel<bf16_t, K_, 16, true><<<grid, 256, 0, st>>>(p)) }
            else { SSM_DISPATCH_KPL(kpl, sens_kernel<bf16_t, K_, 0, true><<<grid, 256, 0, st>>>(p)) }
        }
        return hipGetLastError();
    }
    if (dtype == 0) {
        if (n16) { SSM_DISPATCH_KPL(kpl, sens_kernel<float, K_, 16><<<grid, 256, 0, st>>>(p)) }
        else { SSM_DISPATCH_KPL(kpl, sens_kernel<float, K_, 0><<<grid, 256, 0, st>>>(p)) }
    } else {
        if (n16) { SSM_DISPATCH_KPL(kpl, sens_kernel<bf16_t, K_, 16><<<grid, 256, 0, st>>>(p)) }
        else { SSM_DISPATCH_KPL(kpl, sens_kernel<bf16_t, K_, 0><<<grid, 256, 0, st>>>(p)) }
    }
    return hipGetLastError();
}

hipError_t launch_sens_rows_edge(const SensRowsParams& p, bool tail, int dtype, hipStream_t st) {
    const int total = p.B * p.D * p.R, blocks = (total + 255) / 256;
    if (dtype == 0) {
        if (tail) sens_rows_edge_kernel<float, true><<<blocks, 256, 0, st>>>(p);
        else sens_rows_edge_kernel<float, false><<<blocks, 256, 0, st>>>(p);
    } else {
        if (tail) sens_rows_edge_kernel<bf16_t, true><<<blocks, 256, 0, st>>>(p);
        else sens_rows_edge_kernel<bf16_t, false><<<blocks, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_sens_rows(const SensRowsParams& pin, int dtype, hipStream_t st) {
    if (pin.R < 1 || pin.R > kSensRowsMax || pin.N > 16) return hipErrorInvalidValue;
    SensRowsParams p = pin;
    p.tiles_per_wg = sens_tiles_per_wg(p.ntiles);
    dim3 grid((p.D + 15) / 16, p.B, (p.ntiles + p.tiles_per_wg - 1) / p.tiles_per_wg);
    const bool n16 = p.N == 16;
    if (dtype == 0) {
        if (n16) sens_rows_kernel<float, 16><<<grid, 256, 0, st>>>(p);
        else sens_rows_kernel<float, 0><<<grid, 256, 0, st>>>(p);
    } else {
        if (n16) sens_rows_kernel<bf16_t, 16><<<grid, 256, 0, st>>>(p);
        else sens_rows_kernel<bf16_t, 0><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}

}  // namespace ssm
