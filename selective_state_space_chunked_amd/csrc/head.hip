// Selective scan with one scalar transition per head, in the chunked matrix
// form on the matrix cores (S3M page, section 4.1: the discretisation merged
// with a matrix multiply).  Head h owns channels d = h*P + p (p < P) and a
// state matrix H_t (N x P):
//   a_t = exp(delta_t A_h),  H_t = a_t H_{t-1} + B_t (delta_t x_t)^T,  y_t = H_t^T C_t.
// Within a chunk of T = 64 steps, with s_t = A_h * (delta_0 + ... + delta_t)
// (inclusive, inside the chunk):
//   Y = (G o Lm) (diag(delta) X) + diag(e^s) C H_in,   G = C B^T (T x T),
//   Lm[t][u] = e^(s_t - s_u) for u <= t, else 0,
//   H_out = e^(s_{T-1}) H_in + B^T diag(w) X,         w_u = e^(s_{T-1} - s_u) delta_u,
// where X (T x P), B, C (T x N) are the chunk's rows.  Every product is a dense
// contraction, done with v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).
// Three passes: the chunk-local end states (H_in = 0) and decays; a chain over
// the chunks of each (batch, head) that turns them into entering states; the
// outputs.
//
// MFMA 16x16x4 f32 lane layout (wave64): the A operand (16 x 4) has A[i][k] in
// lane i + 16k, the B operand (4 x 16) B[k][j] in lane j + 16k, and the 16 x 16
// result D[i][j] in register i % 4 of lane j + 16 (i / 4).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kHT = 64;          // chunk length (steps)
constexpr int kHPad = kHT + 1;   // LDS row of one chunk (+1 spreads the rows over banks)

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS layout (float offsets) of a chunk for P channels and N states: delta and
// s (T each), x as [p][u] rows of T + 1, B and C as [u][n] rows of N + 1, the
// entering state as [n][p] rows of P + 1, and each wave's 16 rows of M.
struct HeadLds {
    int dl, s, sx, sB, sC, sH, sM, total;
};
__host__ __device__ inline HeadLds head_lds(int P, int N, bool out) {
    HeadLds o;
    o.dl = 0;
    o.s = kHT;
    o.sx = 2 * kHT;
    o.sB = o.sx + P * kHPad;
    o.sC = o.sB + kHT * (N + 1);
    o.sH = o.sC + (out ? kHT * (N + 1) : 0);
    o.sM = o.sH + (out ? N * (P + 1) : 0);
    o.total = o.sM + (out ? 4 * 16 * kHPad : 0);
    return o;
}

struct HeadTile {
    int b, hh, c, t0, nval;   // batch row, head, chunk, first step, steps in the chunk
};
__device__ __forceinline__ HeadTile head_tile(const HeadParams& p) {
    HeadTile q;
    q.c = blockIdx.x;
    q.hh = blockIdx.y;
    q.b = blockIdx.z;
    q.t0 = q.c * kHT;
    q.nval = min(kHT, p.L - q.t0);
    return q;
}

// Stage the chunk: delta (T), x as [p][u] (P rows of T), B and C as [u][n]
// (T rows of N); steps past the end are zero.  s[u] = A * (inclusive prefix sum
// of delta) in fp32, by one wave (a 64-lane scan: DPP within rows of 16, then
// the row totals).
template <typename T>
__device__ __forceinline__ void head_stage(const HeadParams& p, const HeadTile& q, float* dl, float* sx, float* sB,
                                           float* sC, float* s, bool needC) {
    const int tid = threadIdx.x, P = p.P, N = p.N;
    const T* delta = (const T*)p.delta + (int64_t)q.b * p.sdelta[0] + (int64_t)q.hh * p.sdelta[1] + q.t0;
    for (int u = tid; u < kHT; u += 256) dl[u] = u < q.nval ? to_f32(delta[u]) : 0.0f;
    const T* xb = (const T*)p.x + (int64_t)q.b * p.sx[0] + (int64_t)q.hh * P * p.sx[1] + q.t0;
    for (int e = tid; e < P * kHT; e += 256) {
        const int pp = e / kHT, u = e - pp * kHT;
        sx[pp * kHPad + u] = u < q.nval ? to_f32(xb[(int64_t)pp * p.sx[1] + u]) : 0.0f;
    }
    const T* bb = (const T*)p.Bm + (int64_t)q.b * p.sBm[0] + (int64_t)q.t0 * p.sBm[2];
    const T* cb = (const T*)p.C + (int64_t)q.b * p.sC[0] + (int64_t)q.t0 * p.sC[2];
    for (int e = tid; e < kHT * N; e += 256) {
        const int u = e / N, n = e - u * N;
        const bool v = u < q.nval;
        sB[u * (N + 1) + n] = v ? to_f32(bb[(int64_t)u * p.sBm[2] + n]) : 0.0f;
        if (needC) sC[u * (N + 1) + n] = v ? to_f32(cb[(int64_t)u * p.sC[2] + n]) : 0.0f;
    }
    __syncthreads();
    if (tid < 64) {   // prefix sum of delta over the chunk (wave 0, lane = step)
        float v = dl[tid];
        v += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, v);
        // carry the totals of the earlier 16-lane rows (lane 15 of each row)
        const float r0 = __shfl(v, 15), r1 = __shfl(v, 31), r2 = __shfl(v, 47);
        const int row = tid >> 4;
        v += (row > 0 ? r0 : 0.0f) + (row > 1 ? r1 : 0.0f) + (row > 2 ? r2 : 0.0f);
        s[tid] = p.A[(int64_t)q.hh * p.sA] * v;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// pass 1: chunk-local end state S = B^T diag(w) X (N x P) and decay e^(s_{T-1})
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void head_state_kernel(HeadParams p) {
    extern __shared__ float lds[];
    const int P = p.P, N = p.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const HeadLds o = head_lds(P, N, false);
    float *dl = lds + o.dl, *s = lds + o.s, *sx = lds + o.sx, *sB = lds + o.sB;
    const HeadTile q = head_tile(p);
    head_stage<T>(p, q, dl, sx, sB, nullptr, s, false);
    const float sT = s[kHT - 1];
    const int ntiles = (N / 16) * (P / 16);
    float* S = p.state + (((size_t)q.b * p.H + q.hh) * p.nchunks + q.c) * (size_t)N * P;
    for (int tile = wave; tile < ntiles; tile += 4) {   // uniform per wave
        const int n0 = 16 * (tile / (P / 16)), p0 = 16 * (tile % (P / 16));
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int kk = 0; kk < kHT / 4; ++kk) {
            const int u = 4 * kk + (lane >> 4);
            const float w = __expf(sT - s[u]) * dl[u];
            const float a = sB[u * (N + 1) + n0 + (lane & 15)] * w;   // A[n][u] = B[u][n] w_u
            const float bx = sx[(p0 + (lane & 15)) * kHPad + u];     // B[u][p] = X[u][p]
            acc = mfma4(a, bx, acc);
        }
        // D[n][p]: register r of lane l holds n = n0 + 4 (l / 16) + r, p = p0 + l % 16
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(size_t)(n0 + 4 * (lane >> 4) + r) * P + p0 + (lane & 15)] = acc[r];
    }
    if (threadIdx.x == 0) p.decay[((size_t)q.b * p.H + q.hh) * p.nchunks + q.c] = __expf(sT);
}

// ---------------------------------------------------------------------------
// pass 2: entering states.  One thread per (batch, head, n, p) element: walk the
// chunks in order, H_in(c) = state entering chunk c, H_in(c+1) = decay_c H_in(c)
// + S_c; the local states are overwritten with the entering states; the state
// after the last chunk goes to h_last, and the entering states to the
// checkpoints (B, D, nchunks, N) when requested.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void head_chain_kernel(HeadParams p) {
    const int P = p.P, N = p.N;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)p.B * p.H * N * P) return;
    const int64_t bh = i / ((int64_t)N * P);
    const int e = (int)(i - bh * N * P), n = e / P, pp = e - n * P;
    const int b = (int)(bh / p.H), hh = (int)(bh - (int64_t)b * p.H);
    const int64_t seq = (int64_t)b * p.H * P + (int64_t)hh * P + pp;   // channel row (b, d = h*P + p)
    float h = p.h0 ? p.h0[seq * N + n] : 0.0f;
    float* S = p.state + (size_t)bh * p.nchunks * N * P + e;
    const float* dec = p.decay + (size_t)bh * p.nchunks;
    for (int c = 0; c < p.nchunks; ++c) {
        const float loc = S[(size_t)c * N * P];
        S[(size_t)c * N * P] = h;
        if (p.ckpt) p.ckpt[(seq * p.nchunks + c) * N + n] = h;
        h = fmaf(dec[c], h, loc);
    }
    if (p.h_last) p.h_last[seq * N + n] = h;
}

// ---------------------------------------------------------------------------
// pass 3: outputs.  Wave w computes the 16 steps t = 16w .. 16w+15 of every p:
//   row block of G = C B^T (16 x T), masked and scaled in registers to
//   M[t][u] = G[t][u] e^(s_t - s_u) delta_u (u <= t), written to LDS and read back
//   as A operands; Y = M X + (e^s C) H_in.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void head_out_kernel(HeadParams p) {
    extern __shared__ float lds[];
    const int P = p.P, N = p.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const HeadLds o = head_lds(P, N, true);
    float *dl = lds + o.dl, *s = lds + o.s, *sx = lds + o.sx, *sB = lds + o.sB, *sC = lds + o.sC;
    float* sH = lds + o.sH;   // H_in as [n][p], rows of P + 1
    const HeadTile q = head_tile(p);
    {
        const float* Hin = p.state + (((size_t)q.b * p.H + q.hh) * p.nchunks + q.c) * (size_t)N * P;
        for (int e = threadIdx.x; e < N * P; e += 256) sH[(e / P) * (P + 1) + e % P] = Hin[e];
    }
    head_stage<T>(p, q, dl, sx, sB, sC, s, true);
    const int t0 = 16 * wave;
    if (t0 >= q.nval) return;   // whole waves past the end (no barrier follows)
    // G rows t0.., all 64 columns: 4 column tiles, K = N
    f4 g[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        g[jt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int kk = 0; kk < N / 4; ++kk) {
            const int n = 4 * kk + (lane >> 4);
            const float a = sC[(t0 + (lane & 15)) * (N + 1) + n];      // A[t][n] = C[t][n]
            const float bb = sB[(16 * jt + (lane & 15)) * (N + 1) + n]; // B[n][u] = B[u][n]
            g[jt] = mfma4(a, bb, g[jt]);
        }
    }
    // mask, decay and delta: register r of lane l holds t = t0 + 4 (l/16) + r, u = 16 jt + l % 16
    float* Mw = lds + o.sM + wave * 16 * kHPad;   // this wave's rows of M
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        const int u = 16 * jt + (lane & 15);
        const float su = s[u], du = dl[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tr = 4 * (lane >> 4) + r, t = t0 + tr;
            const float m = u <= t ? g[jt][r] * __expf(s[t] - su) * du : 0.0f;
            Mw[tr * kHPad + u] = m;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done (lgkmcnt 0) before the reads below
    __builtin_amdgcn_wave_barrier();
    const float es = __expf(s[t0 + (lane & 15)]);   // e^(s_t) for the A operand rows
    for (int pt = 0; pt < P / 16; ++pt) {
        const int p0 = 16 * pt;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // intra-chunk: K = T
#pragma unroll 4
        for (int kk = 0; kk < kHT / 4; ++kk) {
            const int u = 4 * kk + (lane >> 4);
            acc = mfma4(Mw[(lane & 15) * kHPad + u], sx[(p0 + (lane & 15)) * kHPad + u], acc);
        }
        // carried state: K = N
        for (int kk = 0; kk < N / 4; ++kk) {
            const int n = 4 * kk + (lane >> 4);
            const float a = sC[(t0 + (lane & 15)) * (N + 1) + n] * es;   // e^(s_t) C[t][n]
            acc = mfma4(a, sH[n * (P + 1) + p0 + (lane & 15)], acc);
        }
        // D[t][p]: lane l, register r: t = t0 + 4 (l/16) + r, p = p0 + l % 16
        const int pp = p0 + (lane & 15), tb = t0 + 4 * (lane >> 4);
        T* yrow = (T*)p.y + (int64_t)q.b * p.sy[0] + ((int64_t)q.hh * P + pp) * p.sy[1] + q.t0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tb + r < q.nval) yrow[tb + r] = from_f32<T>(acc[r]);
    }
}

// gdelta of the head form from the per-channel step-size gradients: the sum over
// the head's P channels, in channel order.  gdc (B, D, L) fp32, out (B, H, L).
template <typename T>
__global__ __launch_bounds__(256) void head_gdelta_kernel(const float* __restrict__ gdc, T* __restrict__ out, int B,
                                                          int H, int P, int L) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)B * H * L) return;
    const int64_t bh = i / L;
    const int t = (int)(i - bh * L);
    const float* src = gdc + bh * P * L + t;
    float acc = 0.0f;
    for (int pp = 0; pp < P; ++pp) acc += src[(int64_t)pp * L];
    out[i] = from_f32<T>(acc);
}
// gA[h] = sum over the head's channels p and states n of gA_dn[h*P + p][n], in order
__global__ __launch_bounds__(64) void head_ga_kernel(const float* __restrict__ ga_dn, float* __restrict__ out, int H,
                                                     int P, int N) {
    const int hh = blockIdx.x * 64 + threadIdx.x;
    if (hh >= H) return;
    float acc = 0.0f;
    for (int e = 0; e < P * N; ++e) acc += ga_dn[(int64_t)hh * P * N + e];
    out[hh] = acc;
}

hipError_t launch_head_fwd(const HeadParams& p, int dtype, hipStream_t st) {
    if (p.P % 16 || p.P > 64 || p.N % 16 || p.N > 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.nchunks, (unsigned)p.H, (unsigned)p.B);
    const size_t l1 = head_lds(p.P, p.N, false).total * sizeof(float), l3 = head_lds(p.P, p.N, true).total * sizeof(float);
    if (dtype == 0) head_state_kernel<float><<<grid, 256, l1, st>>>(p);
    else head_state_kernel<bf16_t><<<grid, 256, l1, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)p.B * p.H * p.N * p.P;
    head_chain_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p);
    if ((e = hipGetLastError()) != hipSuccess || !p.y) return e;
    if (dtype == 0) head_out_kernel<float><<<grid, 256, l3, st>>>(p);
    else head_out_kernel<bf16_t><<<grid, 256, l3, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_reduce(const float* gdc, void* gdelta, const float* ga_dn, float* gA, int B, int H, int P,
                              int N, int L, int dtype, hipStream_t st) {
    if (gdelta) {
        const int64_t n = (int64_t)B * H * L;
        if (dtype == 0)
            head_gdelta_kernel<float><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(gdc, (float*)gdelta, B, H, P, L);
        else
            head_gdelta_kernel<bf16_t><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(gdc, (bf16_t*)gdelta, B, H, P, L);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (gA) {
        head_ga_kernel<<<(unsigned)((H + 63) / 64), 64, 0, st>>>(ga_dn, gA, H, P, N);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace ssm
