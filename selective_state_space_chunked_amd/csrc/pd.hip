// PD-transition scan: preimage tables, chunk chains and the selection copy
// (kernel templates in pd.hpp).
#include "pd.hpp"

namespace ssm {

// preimage lists: pre[(h*K+k)*N*N + i*N + r] = r-th column j (ascending) with
// dict[h,k,j] == i, padded with 0; cnt[(h*K+k)*N + i] = number of such columns.
__global__ void pd_prep_kernel(const int32_t* __restrict__ dict, int64_t sdh, int64_t sdk, int8_t* __restrict__ pre,
                               int32_t* __restrict__ cnt, int H, int K, int N) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= H * K * N) return;
    const int hk = idx / N, i = idx - hk * N;
    const int32_t* col = dict + (int64_t)(hk / K) * sdh + (int64_t)(hk % K) * sdk;   // entry k of head h
    int c = 0;
    // entries outside [0, N) are clamped exactly as pd_load_tables clamps them, so the
    // gather lists and the compositions see the same dictionary
    for (int j = 0; j < N; ++j)
        if (min(max(col[j], 0), N - 1) == i) pre[(size_t)hk * N * N + i * N + c++] = (int8_t)j;
    for (int r = c; r < N; ++r) pre[(size_t)hk * N * N + i * N + r] = 0;
    cnt[idx] = c;
}

// Chunk chains, one workgroup (16 rows of 16 lanes, lane = state) per
// (batch, head), in three phases so the serial depth is about 3 * G / 16
// links instead of G:
//   1. row r composes the chunk maps of its range [r P, (r+1) P) into one map;
//   2. row 0 chains the 16 range maps from the sequence's initial value,
//      leaving each range's entering value in LDS;
//   3. row r re-runs its range from that value and writes every chunk's
//      entering value.
// Forward maps are h -> P_pi diag(D) h + S (a scatter: the columns j with
// pi(j) = i are visited in ascending order with DPP broadcasts); reverse maps
// are v -> D * v[pi] + R (one gather).
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
    __shared__ float sS[16][16], sD[16][16], sH[16][16];
    __shared__ int sPi[16][16];
    const int s = blockIdx.x, row = threadIdx.x >> 4, i = threadIdx.x & 15;
    const int N = p.N, G = p.G;
    const bool nl = i < N;
    const int ic = nl ? i : N - 1;
    const int P = (G + 15) / 16;
    const int g0 = min(row * P, G), g1 = min(g0 + P, G);
    const size_t base = (size_t)s * G * N;
    // phase 1: compose the chunk maps of the range, later chunk applied last:
    // pi <- pi_g[pi], D <- D_g[pi] * D, S <- P_{pi_g} D_g S + S_g
    float S = 0.0f, D = 1.0f;
    int pi = i;
    for (int g = g0; g < g1; ++g) {
        const size_t o = base + (size_t)g * N + ic;
        const float Sg = nl ? p.segS[o] : 0.0f, Dg = nl ? p.segD[o] : 0.0f;
        const int pig = nl ? p.segPi[o] : i;
        S = pd_link_fwd(S, Sg, Dg, pig, i, N);
        if (!nl) S = 0.0f;
        D = row_pull(Dg, pi) * D;
        pi = row_pull_i(pig, pi);
    }
    sS[row][i] = S; sD[row][i] = D; sPi[row][i] = pi;
    __syncthreads();
    // phase 2: chain the range maps
    if (row == 0) {
        float h = (nl && p.h0) ? p.h0[(size_t)s * N + ic] : 0.0f;
        for (int rr = 0; rr < 16; ++rr) {
            sH[rr][i] = h;
            h = pd_link_fwd(h, sS[rr][i], sD[rr][i], sPi[rr][i], i, N);
            if (!nl) h = 0.0f;
        }
    }
    __syncthreads();
    // phase 3: re-run the range from its entering value
    float h = sH[row][i];
    for (int g = g0; g < g1; ++g) {
        const size_t o = base + (size_t)g * N + ic;
        const float Sg = nl ? p.segS[o] : 0.0f, Dg = nl ? p.segD[o] : 0.0f;
        const int pig = nl ? p.segPi[o] : i;
        if (nl) p.carry_in[o] = h;
        h = pd_link_fwd(h, Sg, Dg, pig, i, N);
        if (!nl) h = 0.0f;
    }
}

__global__ __launch_bounds__(256) void pd_combine_rev_kernel(PDParams p) {
    __shared__ float sR[16][16], sD[16][16], sV[16][16];
    __shared__ int sPi[16][16];
    const int s = blockIdx.x, row = threadIdx.x >> 4, j = threadIdx.x & 15;
    const int N = p.N, G = p.G;
    const bool nl = j < N;
    const int jc = nl ? j : N - 1;
    const int P = (G + 15) / 16;
    const int g0 = min(row * P, G), g1 = min(g0 + P, G);
    const size_t base = (size_t)s * G * N;
    // phase 1: F = f_{g0} o ... o f_{g1-1}; composing f_g after the range so far:
    // D <- D_g * D[pi_g], R <- D_g * R[pi_g] + R_g, pi <- pi[pi_g]
    float R = 0.0f, D = 1.0f;
    int pi = j;
    for (int g = g1 - 1; g >= g0; --g) {
        const size_t o = base + (size_t)g * N + jc;
        const float Rg = nl ? p.segS[o] : 0.0f, Dg = nl ? p.segD[o] : 0.0f;
        const int pig = nl ? p.segPi[o] : j;
        R = fmaf(Dg, row_pull(R, pig), Rg);
        D = Dg * row_pull(D, pig);
        pi = row_pull_i(pi, pig);
    }
    sR[row][j] = R; sD[row][j] = D; sPi[row][j] = pi;
    __syncthreads();
    if (row == 0) {
        float v = (nl && p.gh_last) ? p.gh_last[(size_t)s * N + jc] : 0.0f;
        for (int rr = 15; rr >= 0; --rr) {
            sV[rr][j] = v;
            const float vn = fmaf(sD[rr][j], row_pull(v, sPi[rr][j]), sR[rr][j]);
            v = nl ? vn : 0.0f;
        }
    }
    __syncthreads();
    float v = sV[row][j];
    for (int g = g1 - 1; g >= g0; --g) {
        const size_t o = base + (size_t)g * N + jc;
        const float Rg = nl ? p.segS[o] : 0.0f, Dg = nl ? p.segD[o] : 0.0f;
        const int pig = nl ? p.segPi[o] : j;
        if (nl) p.nu_in[o] = v;
        const float vn = fmaf(Dg, row_pull(v, pig), Rg);
        v = nl ? vn : 0.0f;
    }
}

// out = min(max(sel, 0), K - 1): a given selection is reported as the kernels use it
__global__ __launch_bounds__(256) void pd_sel_copy_kernel(const int32_t* __restrict__ sel, int32_t* __restrict__ out,
                                                          size_t n, int K) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = min(max(sel[i], 0), K - 1);
}
hipError_t launch_pd_sel_copy(const int32_t* sel, int32_t* out, size_t n, int K, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    pd_sel_copy_kernel<<<(unsigned)blocks, 256, 0, st>>>(sel, out, n, K);
    return hipGetLastError();
}

hipError_t launch_pd_prep(const PDParams& p, hipStream_t st) {
    const int n = p.H * p.K * p.N;
    pd_prep_kernel<<<(n + 255) / 256, 256, 0, st>>>(p.dict, p.sdict[0], p.sdict[1], p.pre, p.pre_cnt, p.H, p.K, p.N);
    return hipGetLastError();
}
hipError_t launch_pd_combine_fwd(const PDParams& p, hipStream_t st) {
    pd_combine_fwd_kernel<<<p.B * p.H, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_pd_combine_rev(const PDParams& p, hipStream_t st) {
    pd_combine_rev_kernel<<<p.B * p.H, 256, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace ssm
