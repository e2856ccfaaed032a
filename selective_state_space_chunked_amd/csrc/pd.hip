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

// preimage lists: pre[(h*K+k)*N*N + i*N + r] = r-th column j (ascending) with
// dict[h,k,j] == i, or -1; cnt[(h*K+k)*N + i] = number of such columns.
__global__ void pd_prep_kernel(const int32_t* __restrict__ dict, int8_t* __restrict__ pre,
                               int32_t* __restrict__ cnt, int H, int K, int N) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= H * K * N) return;
    const int hk = idx / N, i = idx - hk * N;
    const int32_t* col = dict + (size_t)hk * N;
    int c = 0;
    for (int j = 0; j < N; ++j)
        if (col[j] == i) pre[(size_t)hk * N * N + i * N + c++] = (int8_t)j;
    for (int r = c; r < N; ++r) pre[(size_t)hk * N * N + i * N + r] = -1;
    cnt[idx] = c;
}

struct PDRow {
    int s, b, hh, ch, lane;
    bool act;  // row maps to an existing chunk
};

// Load the head's dictionary and preimage lists into LDS (whole workgroup).
__device__ __forceinline__ void pd_load_tables(const PDParams& p, int hh, int32_t* sdict, int8_t* spre,
                                               int32_t* scnt) {
    const int K = p.K, N = p.N;
    for (int e = threadIdx.x; e < K * N; e += 256) {
        // entries outside [0, N) are a precondition violation; clamping keeps every access in bounds
        sdict[e] = min(max(p.dict[(size_t)hh * K * N + e], 0), N - 1);
        scnt[e] = p.pre_cnt[(size_t)hh * K * N + e];
    }
    for (int e = threadIdx.x; e < K * N * N; e += 256) spre[e] = p.pre[(size_t)hh * K * N * N + e];
    __syncthreads();
}

// h'[i] = b[i] + sum over the preimage of i (ascending j) of v[j]; rows that
// take no step (past L) keep their state.
__device__ __forceinline__ float pd_scatter(float v, float bv, int k, int i, int N, const int8_t* spre,
                                            const int32_t* scnt) {
    const int c = scnt[k * N + i];
    const int8_t* lst = spre + (k * N + i) * N;
    float acc = bv;
    for (int r = 0; r < N; ++r) {
        if (!__any(r < c)) break;
        const int src = r < c ? (int)lst[r] : 0;
        const float pv = row_pull(v, src);
        if (r < c) acc += pv;
    }
    return acc;
}

__device__ __forceinline__ int pd_argmax(const float* __restrict__ lg, int K) {
    int best = 0;
    float bv = lg[0];
    for (int k = 1; k < K; ++k) {
        const float v = lg[k];
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

// ---------------------------------------------------------------------------
// forward.  SUMMARY: chunk composition (pi, D), local state from zero, sel.
// ---------------------------------------------------------------------------
template <bool SUMMARY>
__global__ __launch_bounds__(256) void pd_fwd_kernel(PDParams p) {
    __shared__ int32_t sdict[kPMaxK * 16];
    __shared__ int32_t scnt[kPMaxK * 16];
    __shared__ int8_t spre[kPMaxK * 16 * 16];
    const PDRow r = pd_row(p);
    pd_load_tables(p, r.hh, sdict, spre, scnt);
    if (!r.act) return;
    const int N = p.N, K = p.K, L = p.L;
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
    const int t0 = r.ch * kPChunk;
    for (int blk = 0; blk < kPChunk / 16; ++blk) {
        float yp[16];
        int selbuf = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = t0 + 16 * blk + j;
            yp[j] = 0.0f;
            const bool tv = t < L;
            int k = 0;
            if (tv) {
                if (SUMMARY) k = p.logits ? pd_argmax(p.logits + (srow + t) * K, K) : p.sel_in[srow + t];
                else k = p.sel[srow + t];
                k = min(max(k, 0), K - 1);  // given selections outside [0, K) are clamped
            }
            if (r.lane == j) selbuf = k;
            const size_t o = (srow + (tv ? t : 0)) * N + i;
            const float dv = (tv && nl) ? p.d[o] : 0.0f;
            const float bv = (tv && nl) ? p.b[o] : 0.0f;
            const float hn = pd_scatter(dv * h, bv, k, i, N, spre, scnt);
            if (SUMMARY) {
                // composition with the step, later step applied last
                const int pn = sdict[k * N + pacc];
                const float dsrc = row_pull(dv, pacc);
                if (tv) {
                    Dacc = dsrc * Dacc;
                    pacc = pn;
                }
            }
            if (tv) h = nl ? hn : 0.0f;
            if (!SUMMARY) yp[j] = (tv && nl) ? p.C[o] * h : 0.0f;
        }
        const int t = t0 + 16 * blk + r.lane;
        if (SUMMARY) {
            if (p.sel_out && t < L) p.sel_out[srow + t] = selbuf;
        } else if (p.y) {
            const float ys = row_transpose_sum16(yp);
            if (t < L) p.y[srow + t] = ys;
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
}

// ---------------------------------------------------------------------------
// backward (selection held fixed).  With nu_t = M_t^T lambda_t (nu_L = gh_last):
//   lambda_t = C_t gy_t + nu_{t+1},   nu_t[j] = d_t[j] lambda_t[pi_t(j)],
//   gd_t[j] = lambda_t[pi_t(j)] h_{t-1}[j],  gb_t = lambda_t,  gC_t = gy_t h_t.
// The chunk's states are recomputed from its checkpoint into registers.
// SUMMARY: chunk transition (pi_c, D_c) composed right to left, and the
// adjoint entering the chunk start from zero (R), so nu_start = D_c*nu[pi_c] + R.
// ---------------------------------------------------------------------------
template <bool SUMMARY>
__global__ __launch_bounds__(256) void pd_bwd_kernel(PDParams p) {
    __shared__ int32_t sdict[kPMaxK * 16];
    __shared__ int32_t scnt[kPMaxK * 16];
    __shared__ int8_t spre[kPMaxK * 16 * 16];
    const PDRow r = pd_row(p);
    pd_load_tables(p, r.hh, sdict, spre, scnt);
    if (!r.act) return;
    const int N = p.N, L = p.L;
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
    float hs[kPChunk + 1];
    if (!SUMMARY) {
        hs[0] = nl ? p.ckpt[((size_t)r.s * p.G + r.ch) * N + j] : 0.0f;
#pragma unroll
        for (int q = 0; q < kPChunk; ++q) {
            const int t = t0 + q;
            const bool tv = t < L;
            const int k = tv ? min(max(p.sel[srow + t], 0), p.K - 1) : 0;
            const size_t o = (srow + (tv ? t : 0)) * N + j;
            const float dv = (tv && nl) ? p.d[o] : 0.0f;
            const float bv = (tv && nl) ? p.b[o] : 0.0f;
            const float hn = pd_scatter(dv * hs[q], bv, k, j, N, spre, scnt);
            hs[q + 1] = (tv && nl) ? hn : hs[q];
        }
    }
#pragma unroll
    for (int q = kPChunk - 1; q >= 0; --q) {
        const int t = t0 + q;
        const bool tv = t < L;
        const int k = tv ? min(max(p.sel[srow + t], 0), p.K - 1) : 0;
        const int pj = sdict[k * N + j];
        const size_t o = (srow + (tv ? t : 0)) * N + j;
        const float gyt = tv ? p.gy[srow + t] : 0.0f;
        const float cv = (tv && nl) ? p.C[o] : 0.0f;
        const float dv = (tv && nl) ? p.d[o] : 0.0f;
        const float lam = fmaf(cv, gyt, nu);
        const float lp = row_pull(lam, pj);  // lambda_t[pi_t(j)]
        if (SUMMARY) {
            const int pn = row_pull_i(pacc, pj);
            const float dn = row_pull(Dacc, pj);
            if (tv) {
                pacc = pn;
                Dacc = dn * dv;
                nu = dv * lp;
            }
        } else if (tv) {
            if (nl) {
                if (p.gb) p.gb[o] = lam;
                if (p.gC) p.gC[o] = gyt * hs[q + 1];
                if (p.gd) p.gd[o] = lp * hs[q];
            }
            nu = dv * lp;
        }
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
}

// Chunk chains.  One 16-lane row per (batch, head), lane = state; the chain
// over chunks is sequential, each link a PD-affine map applied to 16 values.
// Forward link: h'[i] = S[i] + sum over columns j (ascending) with pi(j) = i of
// D[j] h[j]; the columns are visited with DPP broadcasts.  Reverse link:
// v'[j] = D[j] v[pi(j)] + R[j], one gather.  The next chunk's summary is
// loaded one link ahead.
__device__ __forceinline__ float pd_link_fwd(float h, float S, float D, int pi, int i, int N) {
    const float v = D * h;
    float acc = S;
    const float pf = __int_as_float(pi);
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        const int pj = __float_as_int(bcast16(pf, jj));
        const float vj = bcast16(v, jj);
        if (jj < N && pj == i) acc += vj;
    }
    return acc;
}

__global__ __launch_bounds__(256) void pd_combine_fwd_kernel(PDParams p) {
    const int s = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int i = threadIdx.x & 15;
    if (s >= p.B * p.H) return;  // whole rows leave together
    const int N = p.N;
    const bool nl = i < N;
    const int ic = nl ? i : N - 1;
    float h = (nl && p.h0) ? p.h0[(size_t)s * N + ic] : 0.0f;
    size_t base = (size_t)s * p.G * N;
    float S = p.segS[base + ic], D = p.segD[base + ic];
    int pi = p.segPi[base + ic];
    for (int g = 0; g < p.G; ++g) {
        float S2 = 0.0f, D2 = 0.0f;
        int pi2 = 0;
        if (g + 1 < p.G) {
            const size_t nb = base + N;
            S2 = p.segS[nb + ic];
            D2 = p.segD[nb + ic];
            pi2 = p.segPi[nb + ic];
        }
        if (nl) p.carry_in[base + ic] = h;
        h = pd_link_fwd(h, S, D, pi, i, N);
        if (!nl) h = 0.0f;
        S = S2; D = D2; pi = pi2;
        base += N;
    }
}
__global__ __launch_bounds__(256) void pd_combine_rev_kernel(PDParams p) {
    const int s = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    if (s >= p.B * p.H) return;
    const int N = p.N;
    const bool nl = j < N;
    const int jc = nl ? j : N - 1;
    float v = (nl && p.gh_last) ? p.gh_last[(size_t)s * N + jc] : 0.0f;
    size_t base = ((size_t)s * p.G + p.G - 1) * N;
    float R = p.segS[base + jc], D = p.segD[base + jc];
    int pi = p.segPi[base + jc];
    for (int g = p.G - 1; g >= 0; --g) {
        float R2 = 0.0f, D2 = 0.0f;
        int pi2 = 0;
        if (g > 0) {
            const size_t nb = base - N;
            R2 = p.segS[nb + jc];
            D2 = p.segD[nb + jc];
            pi2 = p.segPi[nb + jc];
        }
        if (nl) p.nu_in[base + jc] = v;
        const float vn = fmaf(D, row_pull(v, pi), R);
        v = nl ? vn : 0.0f;
        R = R2; D = D2; pi = pi2;
        base -= N;
    }
}

hipError_t launch_pd_prep(const PDParams& p, hipStream_t st) {
    const int n = p.H * p.K * p.N;
    pd_prep_kernel<<<(n + 255) / 256, 256, 0, st>>>(p.dict, p.pre, p.pre_cnt, p.H, p.K, p.N);
    return hipGetLastError();
}
hipError_t launch_pd_fwd(const PDParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.G + 15) / 16, p.B * p.H);
    if (summary) pd_fwd_kernel<true><<<grid, 256, 0, st>>>(p);
    else pd_fwd_kernel<false><<<grid, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_pd_combine_fwd(const PDParams& p, hipStream_t st) {
    const int n = p.B * p.H;
    pd_combine_fwd_kernel<<<(n + 15) / 16, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_pd_bwd(const PDParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.G + 15) / 16, p.B * p.H);
    if (summary) pd_bwd_kernel<true><<<grid, 256, 0, st>>>(p);
    else pd_bwd_kernel<false><<<grid, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_pd_combine_rev(const PDParams& p, hipStream_t st) {
    const int n = p.B * p.H;
    pd_combine_rev_kernel<<<(n + 15) / 16, 256, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace ssm
