// PD-transition scan on gfx950 (Flash PD-SSM page, "Neuer
// Selektionsmechanismus" and "Hardwarebewusste Implementierung"):
//   sel_t = argmax_k logits_t[k] (lowest index among equal maxima),
//   A_t = P_{sel_t} diag(d_t) with P column-one-hot: column j has its one in
//   row pi(j) = dict[h, sel_t, j], so h_t[i] = b_t[i] + sum_{j: pi(j)=i} d_t[j] h_{t-1}[j],
//   y_t = sum_i C_t[i] h_t[i].
//
// Work mapping.  A 16-lane row holds the N states of one (batch, head) over
// one 64-step chunk; a workgroup is 16 consecutive chunks of the same
// (batch, head), so the head's dictionary lives in LDS.  Every chunk is an
// independent parallel unit.  The state update is a scatter-add (pi is not a
// permutation); it is evaluated as a gather: for each target row i the sources
// j with pi(j) = i are listed in ascending j (precomputed once per call), and
// lane i pulls d_t[j] h[j] from lane j with ds_bpermute.  Compositions of PD
// matrices stay PD and are gathers too:
//   (P2 D2)(P1 D1) = P_{pi2[pi1]} diag(D2[pi1] D1),  (P D)^T v = D * v[pi].
// Three phases: the summary pass composes each chunk's transition (pi_c, D_c)
// and local state (and writes sel); the combine pass chains the chunks per
// (batch, head); the main pass re-runs each chunk from its entering state.
//
// Kernel templates and device helpers; the launchers are split over pd.hip
// (tables, chains), pd_fwd.hip, pd_bwd.hip, pd_ste.hip and pd_ste_dense.hip so they compile in
// parallel.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kPChunk = 64;
constexpr int kPMaxK = 64;

// lane i of the row reads v from lane src (0..15) of the same row
__device__ __forceinline__ float row_pull(float v, int src) {
    const int lane = threadIdx.x & 63;
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & ~15) | src) << 2, __float_as_int(v)));
}
__device__ __forceinline__ int row_pull_i(int v, int src) {
    const int lane = threadIdx.x & 63;
    return __builtin_amdgcn_ds_bpermute(((lane & ~15) | src) << 2, v);
}

struct PDRow {
    int s, b, hh, ch, lane;
    bool act;  // row maps to an existing chunk
};

// A head's tables in LDS: the dictionary, the preimage counts, the preimage
// lists at a fixed 16-byte stride per (entry, target row) so a lane reads its
// whole list with one 16-byte load, and the largest count (the number of
// gather rounds every step needs).
struct PDShared {
    int32_t dict[kPMaxK * 16];
    int32_t cnt[kPMaxK * 16];
    __attribute__((aligned(16))) uint8_t pre[kPMaxK * 16 * 16];
    int maxc;
};

__device__ __forceinline__ void pd_load_tables(const PDParams& p, int hh, PDShared& t) {
    const int K = p.K, N = p.N;
    if (threadIdx.x == 0) t.maxc = 0;
    __syncthreads();
    int m = 0;
    for (int e = threadIdx.x; e < K * N; e += 256) {
        // entries outside [0, N) are a precondition violation; clamping keeps every access in bounds
        t.dict[e] = min(max(p.dict[(int64_t)hh * p.sdict[0] + (int64_t)(e / N) * p.sdict[1] + e % N], 0), N - 1);
        const int c = p.pre_cnt[(size_t)hh * K * N + e];
        t.cnt[e] = c;
        m = max(m, c);
    }
    // list entries are stored as byte offsets (4 * source lane) for ds_bpermute
    for (int e = threadIdx.x; e < K * N * 16; e += 256) {
        const int ki = e >> 4, r = e & 15;
        t.pre[e] = r < N ? (uint8_t)(4 * p.pre[(size_t)hh * K * N * N + ki * N + r]) : 0;
    }
    if (m) atomicMax(&t.maxc, m);
    __syncthreads();
}

// Lane i of the row: acc + sum over the preimage of i under dictionary entry
// k, in ascending column order, of v[j] (v lives in lane j of the row).  RM
// rounds, at least the head's largest preimage.
template <int RM>
__device__ __forceinline__ float pd_gather_sum(float v, float acc, int k, int i, int N, const PDShared& t) {
    const int c = t.cnt[k * N + i];
    const uint4 w = *reinterpret_cast<const uint4*>(t.pre + (k * N + i) * 16);
    const int rowbase = (threadIdx.x & 48) << 2;   // byte offset of this row's lane 0
    // pulls in batches of up to four in flight (bounded register use)
#pragma unroll
    for (int r0 = 0; r0 < RM; r0 += 4) {
        constexpr int B4 = RM < 4 ? RM : 4;
        float pv[B4];
#pragma unroll
        for (int q = 0; q < B4; ++q) {
            const int r = r0 + q;
            const uint32_t word = r < 4 ? w.x : r < 8 ? w.y : r < 12 ? w.z : w.w;
            const int addr = rowbase + (int)((word >> (8 * (r & 3))) & 0xff);
            pv[q] = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(v)));
        }
#pragma unroll
        for (int q = 0; q < B4; ++q) acc += r0 + q < c ? pv[q] : 0.0f;
    }
    return acc;
}

// Run body(integral_constant<int, RM>) with the smallest supported round
// count RM >= the head's largest preimage (uniform for the workgroup).
template <typename F>
__device__ __forceinline__ void pd_with_rounds(int maxc, F&& body) {
    if (maxc <= 2) body(std::integral_constant<int, 2>{});
    else if (maxc <= 4) body(std::integral_constant<int, 4>{});
    else if (maxc <= 6) body(std::integral_constant<int, 6>{});
    else if (maxc <= 8) body(std::integral_constant<int, 8>{});
    else body(std::integral_constant<int, 16>{});
}

template <typename T>
__device__ __forceinline__ int pd_argmax(const T* __restrict__ lg, int K) {
    // 16-byte loads when the row allows; the comparisons run in the same order
    constexpr int V = 16 / sizeof(T);
    if (K % V == 0 && (reinterpret_cast<uintptr_t>(lg) & 15) == 0) {
        int best = 0;
        float bv = 0.0f;
        for (int k0 = 0; k0 < K; k0 += V) {
            const uint4 w = *reinterpret_cast<const uint4*>(lg + k0);
            T e[V];
            __builtin_memcpy(e, &w, 16);
#pragma unroll
            for (int u = 0; u < V; ++u) {
                const float v = to_f32(e[u]);
                if (k0 + u == 0) bv = v;
                else if (v > bv) { bv = v; best = k0 + u; }
            }
        }
        return best;
    }
    int best = 0;
    float bv = to_f32(lg[0]);
    for (int k = 1; k < K; ++k) {
        const float v = to_f32(lg[k]);
        if (v > bv) { bv = v; best = k; }
    }
    return best;
}

__device__ __forceinline__ PDRow pd_row(const PDParams& p) {
    PDRow r;
    r.lane = threadIdx.x & 15;
    r.s = blockIdx.y;
    r.b = r.s / p.H;
    r.hh = r.s - r.b * p.H;
    r.ch = blockIdx.x * 16 + (threadIdx.x >> 4);
    r.act = r.ch < p.G;
    return r;
}

// 16 steps tb.. of state i of an (L, N) slice (fp32 or bf16); steps past L
// read 0.  DENSE: rows of N states back to back, 32-bit offsets from one
// address (constant ones for a compile-time N); otherwise the steps are sl
// elements apart and each step's address is formed in 64 bits.
template <typename T, int NT, bool DENSE>
__device__ __forceinline__ void pd_load16(const T* __restrict__ base, int64_t sl, int tb, int L, int N, int i,
                                          float (&v)[16]) {
    if constexpr (DENSE) {
        const int n = NT ? NT : N;
        const T* __restrict__ q = base + (size_t)tb * n + i;
        if (tb + 16 <= L) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = to_f32(q[j * n]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = tb + j < L ? to_f32(q[j * n]) : 0.0f;
        }
    } else {
        const T* __restrict__ q = base + (int64_t)tb * sl + i;
        if (tb + 16 <= L) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = to_f32(q[(int64_t)j * sl]);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = tb + j < L ? to_f32(q[(int64_t)j * sl]) : 0.0f;
        }
    }
}

// The (b, h) rows of d, b, C (and of the scores): dense, or through the views' strides.
template <typename T, bool DENSE>
__device__ __forceinline__ const T* pd_rowbase(const void* base, const int64_t (&s)[3], const PDRow& r, size_t srow,
                                               int W) {
    if constexpr (DENSE) return (const T*)base + srow * W;
    return (const T*)base + ((int64_t)r.b * s[0] + (int64_t)r.hh * s[1]);
}

// ---------------------------------------------------------------------------
// forward.  SUMMARY: chunk composition (pi, D), local state from zero, sel.
// Each 16-step block first loads everything it needs (lane l takes the
// selection of step l; d, b and C for all 16 steps), then runs the steps.
// ---------------------------------------------------------------------------
template <typename T, bool SUMMARY, int NT, bool DENSE>
__global__ __launch_bounds__(256) void pd_fwd_kernel(PDParams p) {
    __shared__ PDShared tb_;
    const PDRow r = pd_row(p);
    pd_load_tables(p, r.hh, tb_);
    if (!r.act) return;
    pd_with_rounds(tb_.maxc, [&](auto rounds) {
        constexpr int RM = decltype(rounds)::value;
        const int N = NT ? NT : p.N, K = p.K, L = p.L;
        const bool nl = r.lane < N;
        const int i = nl ? r.lane : N - 1;
        const size_t srow = (size_t)r.s * L;
        float h = 0.0f;
        int pacc = i;
        float Dacc = 1.0f;
        if (!SUMMARY) {
            if (p.G > 1) h = p.carry_in[((size_t)r.s * p.G + r.ch) * N + i];
            else if (p.h0) h = p.h0[(size_t)r.s * N + i];
            if (p.ckpt_out && nl) p.ckpt_out[((size_t)r.s * p.G + r.ch) * N + i] = h;
            if (!nl) h = 0.0f;
        }
        const T* dbase = pd_rowbase<T, DENSE>(p.d, p.s_d, r, srow, N);
        const T* bbase = pd_rowbase<T, DENSE>(p.b, p.s_b, r, srow, N);
        const T* cbase = pd_rowbase<T, DENSE>(p.C, p.s_C, r, srow, N);
        const T* lbase = p.logits ? pd_rowbase<T, DENSE>(p.logits, p.s_lg, r, srow, K) : nullptr;
        const int64_t lstep = DENSE ? K : p.s_lg[2];
        const int t0 = r.ch * kPChunk;
        for (int blk = 0; blk < kPChunk / 16; ++blk) {
            const int tb = t0 + 16 * blk;
            const int tl = tb + r.lane;          // the step whose selection this lane loads
            int kl = 0;
            if (tl < L) {
                if (SUMMARY) kl = lbase ? pd_argmax(lbase + (int64_t)tl * lstep, K) : p.sel_in[srow + tl];
                else kl = p.sel[srow + tl];
                kl = min(max(kl, 0), K - 1);   // given selections outside [0, K) are clamped
            }
            if (SUMMARY && p.sel_out && tl < L) p.sel_out[srow + tl] = kl;
            float dv[16], bv[16], cv[16];
            pd_load16<T, NT, DENSE>(dbase, p.s_d[2], tb, L, N, i, dv);
            pd_load16<T, NT, DENSE>(bbase, p.s_b[2], tb, L, N, i, bv);
            if (!SUMMARY) pd_load16<T, NT, DENSE>(cbase, p.s_C[2], tb, L, N, i, cv);
            float yp[16];
    #pragma unroll
            for (int j = 0; j < 16; ++j) {
                const bool tv = tb + j < L;
                const int k = __float_as_int(bcast16(__int_as_float(kl), j));
                const float hn = pd_gather_sum<RM>(dv[j] * h, bv[j], k, i, N, tb_);
                if (SUMMARY) {
                    // composition with the step, later step applied last
                    const int pn = tb_.dict[k * N + pacc];
                    const float dsrc = row_pull(dv[j], pacc);
                    if (tv) {
                        Dacc = dsrc * Dacc;
                        pacc = pn;
                    }
                }
                if (tv) h = nl ? hn : 0.0f;
                if (!SUMMARY) yp[j] = (tv && nl) ? cv[j] * h : 0.0f;
            }
            if (!SUMMARY && p.y) {
                const float ys = row_transpose_sum16(yp);
                if (tl < L) ((T*)p.y)[srow + tl] = from_f32<T>(ys);
            }
        }
        if (!nl) return;
        const size_t so = ((size_t)r.s * p.G + r.ch) * N + i;
        if (SUMMARY) {
            p.segPi[so] = pacc;
            p.segD[so] = Dacc;
            p.segS[so] = h;
        } else if (p.h_last && r.ch == p.G - 1) {
            p.h_last[(size_t)r.s * N + i] = h;
        }

    });
}

// ---------------------------------------------------------------------------
// backward (selection held fixed).  With nu_t = M_t^T lambda_t (nu_L = gh_last):
//   lambda_t = C_t gy_t + nu_{t+1},   nu_t[j] = d_t[j] lambda_t[pi_t(j)],
//   gd_t[j] = lambda_t[pi_t(j)] h_{t-1}[j],  gb_t = lambda_t,  gC_t = gy_t h_t.
// The chunk's states are recomputed from its checkpoint into registers, 16
// steps per batch of loads; the reverse sweep loads its blocks in the same way.
// SUMMARY: chunk transition (pi_c, D_c) composed right to left, and the
// adjoint entering the chunk start from zero (R), so nu_start = D_c*nu[pi_c] + R.
// STE >= 0 (main pass only; 16 = register path for K <= 16): straight-through
// surrogate gradient of the selection (Flash PD-SSM page, gradient
// propagation: hard argmax forward, tempered softmax backward).  With the
// transition read as sum_k w_k P_k diag(d_t),
//   gw[t,k] = sum_j lambda_t[pi_k(j)] d_t[j] h_{t-1}[j],
//   glogits[t,k] = (1/tau) s_k (gw[t,k] - <s, gw[t,:]>),  s = softmax(logits_t / tau).
// Per 16-step block and entry k every lane pulls lambda_t[pi_k(j)] for the 16
// steps and one transpose-reduction over the row leaves gw of step tb + lane
// on that lane; each lane then applies the softmax pull-back to its step.
// ---------------------------------------------------------------------------
// Surrogate selection gradient of one 16-step block; lam[q], z[q] = lambda_t[j]
// and d_t[j] h_{t-1}[j] of step tb + q on lane j.  KR = 16: K <= 16, the
// lane's scores x (preloaded, -inf past K) and its gw stay in registers;
// KR = 0: any K, gw goes through the output array.
template <typename T, int KR>
__device__ __forceinline__ void pd_ste_block(const PDParams& p, const PDShared& tb_, const float (&lam)[16],
                                             const float (&z)[16], const float (&x)[16], size_t srow, int tb,
                                             int N, int j) {
    const int K = p.K, L = p.L;
    const int t = tb + (lane_id() & 15);   // the step whose gw this lane receives
    T* o = (T*)p.glogits + (srow + t) * K;
    const float sc = p.inv_tau * 1.4426950408889634f;  // exp(v / tau) = 2^(v log2(e) / tau)
    if (KR == 16) {
        float g[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            g[k] = 0.0f;
            if (k < K) {                   // uniform
                const int pk = tb_.dict[k * N + j];
                float v[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) v[q] = row_pull(lam[q], pk) * z[q];
                g[k] = row_transpose_sum16(v);
            }
        }
        if (t >= L) return;
        float mx = x[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) mx = fmaxf(mx, x[k]);
        float e[16], zs = 0.0f, dot = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            e[k] = k < K ? exp2f((x[k] - mx) * sc) : 0.0f;
            zs += e[k];
            dot = fmaf(e[k], g[k], dot);
        }
        const float rz = 1.0f / zs;
        dot *= rz;
        constexpr int V = 16 / sizeof(T);   // scores per 16-byte store
        if (K % V == 0 && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
#pragma unroll
            for (int k0 = 0; k0 < 16; k0 += V) {
                if (k0 < K) {
                    T v[V];
#pragma unroll
                    for (int u = 0; u < V; ++u) v[u] = from_f32<T>(e[k0 + u] * rz * (g[k0 + u] - dot) * p.inv_tau);
                    uint4 w;
                    __builtin_memcpy(&w, v, 16);
                    *reinterpret_cast<uint4*>(o + k0) = w;
                }
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (k < K) o[k] = from_f32<T>(e[k] * rz * (g[k] - dot) * p.inv_tau);
        return;
    }
    for (int k = 0; k < K; ++k) {          // uniform
        const int pk = tb_.dict[k * N + j];
        float v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = row_pull(lam[q], pk) * z[q];
        const float g = row_transpose_sum16(v);
        if (t < L) o[k] = from_f32<T>(g);  // gw, replaced by glogits below (fp32 only, see the launcher)
    }
    if (t >= L) return;
    const T* xs = (const T*)p.ste_logits + (srow + t) * K;
    float mx = to_f32(xs[0]);
    for (int k = 1; k < K; ++k) mx = fmaxf(mx, to_f32(xs[k]));
    float zs = 0.0f, dot = 0.0f;
    for (int k = 0; k < K; ++k) {
        const float e = exp2f((to_f32(xs[k]) - mx) * sc);
        zs += e;
        dot = fmaf(e, to_f32(o[k]), dot);
    }
    const float rz = 1.0f / zs;
    dot *= rz;
    for (int k = 0; k < K; ++k) {
        const float e = exp2f((to_f32(xs[k]) - mx) * sc) * rz;
        o[k] = from_f32<T>(e * (to_f32(o[k]) - dot) * p.inv_tau);
    }
}

template <typename T, bool SUMMARY, int NT, int STE, bool DENSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(STE >= 0 ? 2 : 3))) void pd_bwd_kernel(PDParams p) {
    __shared__ PDShared tb_;
    const PDRow r = pd_row(p);
    pd_load_tables(p, r.hh, tb_);
    if (!r.act) return;
    pd_with_rounds(tb_.maxc, [&](auto rounds) {
        constexpr int RM = decltype(rounds)::value;
        const int N = NT ? NT : p.N, K = p.K, L = p.L;
        const bool nl = r.lane < N;
        const int j = nl ? r.lane : N - 1;  // this lane's state index
        const size_t srow = (size_t)r.s * L;
        const int t0 = r.ch * kPChunk;
        float nu = 0.0f;
        int pacc = j;
        float Dacc = 1.0f;
        if (!SUMMARY && nl) {
            if (p.G > 1) nu = p.nu_in[((size_t)r.s * p.G + r.ch) * N + j];
            else if (p.gh_last) nu = p.gh_last[(size_t)r.s * N + j];
        }
        const T* dbase = pd_rowbase<T, DENSE>(p.d, p.s_d, r, srow, N);
        const T* bbase = pd_rowbase<T, DENSE>(p.b, p.s_b, r, srow, N);
        const T* cbase = pd_rowbase<T, DENSE>(p.C, p.s_C, r, srow, N);
        auto sel_of = [&](int tl) { return tl < L ? min(max(p.sel[srow + tl], 0), K - 1) : 0; };
        float hs[kPChunk + 1];
        if (!SUMMARY) {
            hs[0] = nl ? p.ckpt[((size_t)r.s * p.G + r.ch) * N + j] : 0.0f;
    #pragma unroll
            for (int blk = 0; blk < kPChunk / 16; ++blk) {
                const int tb = t0 + 16 * blk;
                const int kl = sel_of(tb + r.lane);
                float dv[16], bv[16];
                pd_load16<T, NT, DENSE>(dbase, p.s_d[2], tb, L, N, j, dv);
                pd_load16<T, NT, DENSE>(bbase, p.s_b[2], tb, L, N, j, bv);
    #pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int k = __float_as_int(bcast16(__int_as_float(kl), q));
                    const float hn = pd_gather_sum<RM>(dv[q] * hs[16 * blk + q], bv[q], k, j, N, tb_);
                    hs[16 * blk + q + 1] = (tb + q < L && nl) ? hn : hs[16 * blk + q];
                }
            }
        }
    #pragma unroll
        for (int blk = kPChunk / 16 - 1; blk >= 0; --blk) {
            const int tb = t0 + 16 * blk;
            const int tl = tb + r.lane;
            const int kl = sel_of(tl);
            const float gyl = tl < L ? to_f32(((const T*)p.gy)[srow + tl]) : 0.0f;
            float xl[16];  // STE == 16: this lane's scores of step tl
            if (STE == 16) {
                const T* xs = (const T*)p.ste_logits + (srow + tl) * p.K;
                constexpr int V = 16 / sizeof(T);   // scores per 16-byte load
                if (tl < L && p.K % V == 0 && (reinterpret_cast<uintptr_t>(xs) & 15) == 0) {
#pragma unroll
                    for (int k0 = 0; k0 < 16; k0 += V) {
                        T e[V];
                        if (k0 < p.K) {
                            const uint4 w = *reinterpret_cast<const uint4*>(xs + k0);
                            __builtin_memcpy(e, &w, 16);
                        }
#pragma unroll
                        for (int u = 0; u < V; ++u) xl[k0 + u] = k0 < p.K ? to_f32(e[u]) : -INFINITY;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 16; ++k) xl[k] = (k < p.K && tl < L) ? to_f32(xs[k]) : -INFINITY;
                }
            }
            float dv[16], cv[16];
            pd_load16<T, NT, DENSE>(dbase, p.s_d[2], tb, L, N, j, dv);
            pd_load16<T, NT, DENSE>(cbase, p.s_C[2], tb, L, N, j, cv);
            const size_t obase = (srow + tb) * N + j;   // step q at obase + q * N
    #pragma unroll
            for (int q = 15; q >= 0; --q) {
                const bool tv = tb + q < L;
                const int k = __float_as_int(bcast16(__int_as_float(kl), q));
                const float gyt = bcast16(gyl, q);
                const int pj = tb_.dict[k * N + j];
                const float lam = fmaf(cv[q], gyt, nu);
                const float lp = row_pull(lam, pj);  // lambda_t[pi_t(j)]
                if (SUMMARY) {
                    const int pn = row_pull_i(pacc, pj);
                    const float dn = row_pull(Dacc, pj);
                    if (tv) {
                        pacc = pn;
                        Dacc = dn * dv[q];
                        nu = dv[q] * lp;
                    }
                } else if (tv) {
                    if (nl) {
                        const size_t o = obase + (size_t)q * N;
                        if (p.gb) ((T*)p.gb)[o] = from_f32<T>(lam);
                        if (p.gC) ((T*)p.gC)[o] = from_f32<T>(gyt * hs[16 * blk + q + 1]);
                        if (p.gd) ((T*)p.gd)[o] = from_f32<T>(lp * hs[16 * blk + q]);
                    }
                    nu = dv[q] * lp;
                }
                if (STE >= 0) {  // keep lambda_t and d_t[j] h_{t-1}[j] of the block (the slots are free now)
                    cv[q] = tv ? lam : 0.0f;
                    dv[q] = (tv && nl) ? dv[q] * hs[16 * blk + q] : 0.0f;
                }
            }
            if (STE >= 0) pd_ste_block<T, STE == 16 ? 16 : 0>(p, tb_, cv, dv, xl, srow, tb, N, j);
        }
        if (!nl) return;
        const size_t so = ((size_t)r.s * p.G + r.ch) * N + j;
        if (SUMMARY) {
            p.segPi[so] = pacc;
            p.segD[so] = Dacc;
            p.segS[so] = nu;
        } else if (p.gh0 && r.ch == 0) {
            p.gh0[(size_t)r.s * N + j] = nu;
        }

    });
}

// the straight-through backward's instantiations (pd_ste.hip, pd_ste_dense.hip)
hipError_t launch_pd_bwd_ste(const PDParams& p, hipStream_t st);
hipError_t launch_pd_bwd_ste_dense(const PDParams& p, hipStream_t st);
hipError_t launch_pd_bwd_ste_views(const PDParams& p, hipStream_t st);

}  // namespace ssm
