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

constexpr int kHT = 64;     // chunk length (steps)
constexpr int kXLd = 68;    // LDS row of a chunk of x, B^T or M: 16-byte aligned rows 4 banks apart

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS row of N states: N + 4 (16-byte aligned rows that start 4 banks apart).
__host__ __device__ inline int ld_rows_i(int N) { return N + 4; }

// LDS layout (float offsets, multiples of 4): delta, s and the state weights w
// (T each), x as [p][u], B and C as [u][n] (B as [n][u] in the state pass), the
// entering state as [p][n], and each wave's 16 rows of M.
struct HeadLds {
    int dl, s, w, sx, sB, sC, sH, sM, total;
};
__host__ __device__ inline HeadLds head_lds(int P, int N, bool out) {
    HeadLds o;
    o.dl = 0;
    o.s = kHT;
    o.w = 2 * kHT;
    o.sx = 3 * kHT;
    o.sB = o.sx + P * kXLd;
    o.sC = o.sB + (out ? kHT * ld_rows_i(N) : N * kXLd);
    o.sH = o.sC + (out ? kHT * ld_rows_i(N) : 0);
    o.sM = o.sH + (out ? P * ld_rows_i(N) : 0);
    o.total = o.sM + (out ? 4 * 16 * kXLd : 0);
    return o;
}

struct HeadTile {
    int b, hh, c, t0, nval;   // batch row, head, chunk, first step, steps in the chunk
};
template <typename Prm>   // HeadParams or HeadBwdParams: grid (chunk, head, batch)
__device__ __forceinline__ HeadTile head_tile(const Prm& p) {
    HeadTile q;
    q.c = blockIdx.x;
    q.hh = blockIdx.y;
    q.b = blockIdx.z;
    q.t0 = q.c * kHT;
    q.nval = min(kHT, p.L - q.t0);
    return q;
}

__device__ __forceinline__ void unpack16(const uint4& r, float (&f)[8]) {   // 8 bf16
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4& r, float (&f)[4]) {   // 4 fp32
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}

// An R x K tile (row r at base + r * rs, K contiguous elements; R * K <= 4096,
// K a multiple of 16) moves to LDS as fp32, dst[r * ld + k] (dst[k * ld + r]
// when tr), zero outside rows < vr and columns < vk, by 256 threads (tid < 256).  Whole tiles with 16-byte
// aligned rows (VEC) go in two steps: tile_fetch issues a thread's 16-byte
// loads into 16 registers, so that the loads of several tiles are in flight
// together, and tile_put unpacks and writes them.  Otherwise tile_put loads
// and writes the tile by itself, 16 elements a thread, all loads first.  No
// branch guards a load: an index past the tile is clamped to its last element
// (the same value goes to the same place twice) and a masked one reads the
// first element and writes zero.  Row and column of a flat index come from a
// float product with the reciprocal of the row length: exact for indices
// below 2^12 and rows of at most 64.
template <typename T>
struct TileSrc {
    const T* base;
    int64_t rs;
    int R, K, vr, vk;
};
__device__ __forceinline__ int tile_row(int i, float inv) { return (int)(((float)i + 0.5f) * inv); }

template <typename T, bool VEC>
__device__ __forceinline__ void tile_fetch(const TileSrc<T>& ts, float (&v)[16], int tid) {
    if constexpr (VEC) {
        constexpr int E = 16 / (int)sizeof(T);
        const int kp = ts.K / E, np = ts.R * kp;
        const float inv = 1.0f / (float)kp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (256 * j >= np) break;   // uniform
            const int i = min(tid + 256 * j, np - 1);
            const int r = tile_row(i, inv), k = (i - r * kp) * E;
            const uint4 raw = *(const uint4*)(ts.base + (int64_t)r * ts.rs + k);
            v[4 * j] = __uint_as_float(raw.x); v[4 * j + 1] = __uint_as_float(raw.y);
            v[4 * j + 2] = __uint_as_float(raw.z); v[4 * j + 3] = __uint_as_float(raw.w);
        }
    }
}

template <typename T, bool VEC>
__device__ __forceinline__ void tile_put(const TileSrc<T>& ts, const float (&v)[16], float* __restrict__ dst, int ld,
                                         bool tr, int tid) {
    if constexpr (VEC) {
        constexpr int E = 16 / (int)sizeof(T);
        const int kp = ts.K / E, np = ts.R * kp;
        const float inv = 1.0f / (float)kp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (256 * j >= np) break;   // uniform
            const int i = min(tid + 256 * j, np - 1);
            const int r = tile_row(i, inv), k = (i - r * kp) * E;
            float f[E];
            if constexpr (E == 8) {   // 8 bf16
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w = __float_as_uint(v[4 * j + q]);
                    f[2 * q] = __uint_as_float(w << 16);
                    f[2 * q + 1] = __uint_as_float(w & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) f[q] = v[4 * j + q];
            }
            if (tr) {
#pragma unroll
                for (int q = 0; q < E; ++q) dst[(k + q) * ld + r] = f[q];
            } else {
#pragma unroll
                for (int q = 0; q < E; q += 4)
                    *(float4*)&dst[r * ld + k + q] = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
            }
        }
    } else {
        const float inv = 1.0f / (float)ts.K;
        const int ne = ts.R * ts.K;
        float u[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (256 * j >= ne) break;   // uniform
            const int i = min(tid + 256 * j, ne - 1);
            const int r = tile_row(i, inv), k = i - r * ts.K;
            u[j] = to_f32(ts.base[r < ts.vr && k < ts.vk ? (int64_t)r * ts.rs + k : 0]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (256 * j >= ne) break;   // uniform
            const int i = min(tid + 256 * j, ne - 1);
            const int r = tile_row(i, inv), k = i - r * ts.K;
            dst[tr ? k * ld + r : r * ld + k] = r < ts.vr && k < ts.vk ? u[j] : 0.0f;
        }
    }
}

// The chunk's tiles: delta (T), x as [p][u] (P rows of T), B (and C) as [u][n];
// steps past the end are zero.  head_fetch issues the loads (all of them for
// whole aligned tiles); head_put writes LDS, then wave 0 forms s[u] = A * the
// inclusive prefix sum of delta over the chunk in fp32 (a 64-lane scan: DPP
// within rows of 16, then the row totals) and the state weights
// w[u] = e^(s_{T-1} - s_u) delta_u.
template <typename T>
struct HeadRegs {
    float x[16], b[16], c[16], dv, A;
    TileSrc<T> tx, tb, tc;
};
template <typename T, bool VEC>
__device__ __forceinline__ void head_fetch(const HeadParams& p, const HeadTile& q, bool needC, HeadRegs<T>& g) {
    const int tid = threadIdx.x, P = p.P, N = p.N;
    const T* delta = (const T*)p.delta + (int64_t)q.b * p.sdelta[0] + (int64_t)q.hh * p.sdelta[1] + q.t0;
    g.dv = to_f32(delta[min(tid, q.nval - 1)]);
    g.A = p.A[(int64_t)q.hh * p.sA];
    g.tx = TileSrc<T>{(const T*)p.x + (int64_t)q.b * p.sx[0] + (int64_t)q.hh * P * p.sx[1] + q.t0, p.sx[1], P, kHT,
                      P, q.nval};
    g.tb = TileSrc<T>{(const T*)p.Bm + (int64_t)q.b * p.sBm[0] + (int64_t)q.t0 * p.sBm[2], p.sBm[2], kHT, N, q.nval,
                      N};
    g.tc = TileSrc<T>{(const T*)p.C + (int64_t)q.b * p.sC[0] + (int64_t)q.t0 * p.sC[2], p.sC[2], kHT, N, q.nval, N};
    tile_fetch<T, VEC>(g.tx, g.x, tid);
    tile_fetch<T, VEC>(g.tb, g.b, tid);
    if (needC) tile_fetch<T, VEC>(g.tc, g.c, tid);
}
template <typename T, bool VEC>
__device__ __forceinline__ void head_put(const HeadParams& p, const HeadTile& q, const HeadRegs<T>& g, float* dl,
                                         float* s, float* w, float* sx, float* sB, float* sC, int ldb, bool trB) {
    const int tid = threadIdx.x;
    tile_put<T, VEC>(g.tx, g.x, sx, kXLd, false, tid);
    tile_put<T, VEC>(g.tb, g.b, sB, ldb, trB, tid);
    if (sC) tile_put<T, VEC>(g.tc, g.c, sC, ldb, false, tid);
    if (tid < kHT) {   // wave 0, lane = step
        const float dv = tid < q.nval ? g.dv : 0.0f;
        float v = dv;
        v += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, v);
        v += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, v);
        // carry the totals of the earlier 16-lane rows (lane 15 of each row)
        const float r0 = __shfl(v, 15), r1 = __shfl(v, 31), r2 = __shfl(v, 47);
        const int row = tid >> 4;
        v += (row > 0 ? r0 : 0.0f) + (row > 1 ? r1 : 0.0f) + (row > 2 ? r2 : 0.0f);
        const float su = g.A * v;
        const float sT = __shfl(su, kHT - 1);
        dl[tid] = dv;
        s[tid] = su;
        // the backward's state pass (x = gy, B = C) weighs step u by e^(s_u)
        w[tid] = p.bstate ? __expf(su) : __expf(sT - su) * dv;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// pass 1: chunk-local end state, as S^T = X^T diag(w) B (P x N; zero entering
// state), stored [p][n], and the chunk decay e^(s_{T-1}).
// ---------------------------------------------------------------------------
template <typename T, bool VEC>
__device__ __forceinline__ void head_state_body(const HeadParams& p, const HeadTile& q, float* lds) {
    const int P = p.P, N = p.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const HeadLds o = head_lds(P, N, false);
    float *dl = lds + o.dl, *s = lds + o.s, *w = lds + o.w, *sx = lds + o.sx, *sB = lds + o.sB;
    HeadRegs<T> g;
    head_fetch<T, VEC>(p, q, false, g);
    head_put<T, VEC>(p, q, g, dl, s, w, sx, sB, nullptr, kXLd, true);
    const int ntiles = (N / 16) * (P / 16), i = lane & 15, j = lane >> 4;
    float* S = p.state + (((size_t)q.b * p.H + q.hh) * p.nchunks + q.c) * (size_t)N * P;
    for (int tile = wave; tile < ntiles; tile += 4) {   // uniform per wave
        const int p0 = 16 * (tile / (N / 16)), n0 = 16 * (tile % (N / 16));
        // k-group j of every MFMA covers steps u = 16 j .. 16 j + 15 in turn, so a lane reads
        // 16 consecutive steps of its row: A[p][u] = X[u][p], B[u][n] = w_u B[u][n]
        const float* xa = sx + (p0 + i) * kXLd + 16 * j;
        const float* ba = sB + (n0 + i) * kXLd + 16 * j;
        const float* wa = w + 16 * j;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const float4 a4 = *(const float4*)(xa + 4 * k4), b4 = *(const float4*)(ba + 4 * k4),
                         w4 = *(const float4*)(wa + 4 * k4);
            acc = mfma4(a4.x, b4.x * w4.x, acc);
            acc = mfma4(a4.y, b4.y * w4.y, acc);
            acc = mfma4(a4.z, b4.z * w4.z, acc);
            acc = mfma4(a4.w, b4.w * w4.w, acc);
        }
        // D[p][n]: register r of lane l holds p = p0 + 4 (l / 16) + r, n = n0 + l % 16
#pragma unroll
        for (int r = 0; r < 4; ++r) S[(size_t)(p0 + 4 * (lane >> 4) + r) * N + n0 + (lane & 15)] = acc[r];
    }
    if (threadIdx.x == 0) p.decay[((size_t)q.b * p.H + q.hh) * p.nchunks + q.c] = __expf(s[kHT - 1]);
}
template <typename T>
__global__ __launch_bounds__(256) void head_state_kernel(HeadParams p) {
    extern __shared__ __align__(16) float lds[];
    const HeadTile q = head_tile(p);
    if (p.vx && p.vb && q.nval == kHT) head_state_body<T, true>(p, q, lds);   // uniform per block
    else head_state_body<T, false>(p, q, lds);
}

// ---------------------------------------------------------------------------
// pass 2: entering states.  One thread per (batch, head, p, n) element walks
// the chunks in order: H_in(0) = h0, H_in(c+1) = decay_c H_in(c) + S_c.  The
// entering states go to the checkpoints (B, D, nchunks, N) when requested,
// else over the local states; the state after the last chunk to h_last.
// ---------------------------------------------------------------------------
constexpr int kChainGroup = 16;   // chunks whose loads are in flight together
__global__ __launch_bounds__(256) void head_chain_kernel(HeadParams p) {
    const int P = p.P, N = p.N, NP = N * P, nch = p.nchunks;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)p.B * p.H * NP) return;
    const int64_t bh = i / NP;
    const int e = (int)(i - bh * NP), pp = e / N, n = e - pp * N;
    const int b = (int)(bh / p.H), hh = (int)(bh - (int64_t)b * p.H);
    const int64_t seq = (int64_t)b * p.H * P + (int64_t)hh * P + pp;   // channel row (b, d = h*P + p)
    float h = p.h0 ? p.h0[seq * N + n] : 0.0f;
    const float* S = p.state + (size_t)bh * nch * NP + e;
    const float* dec = p.decay + (size_t)bh * nch;
    float* out = p.ckpt ? p.ckpt + seq * nch * N + n : p.state + (size_t)bh * nch * NP + e;
    const int64_t os = p.ckpt ? N : NP;
    for (int c0 = 0; c0 < nch; c0 += kChainGroup) {
        float loc[kChainGroup], dc[kChainGroup];
#pragma unroll
        for (int j = 0; j < kChainGroup; ++j)
            if (c0 + j < nch) {
                loc[j] = S[(size_t)(c0 + j) * NP];
                dc[j] = dec[c0 + j];
            }
#pragma unroll
        for (int j = 0; j < kChainGroup; ++j)
            if (c0 + j < nch) {
                out[(c0 + j) * os] = h;
                h = fmaf(dc[j], h, loc[j]);
            }
    }
    if (p.h_last) p.h_last[seq * N + n] = h;
}

// ---------------------------------------------------------------------------
// pass 3: outputs.  Each wave computes one block of 16 steps t = t0 .. t0+15 for
// every p: the row block of G = C B^T up to the diagonal block, masked and
// scaled in registers to M[t][u] = G[t][u] e^(s_t - s_u) delta_u (u <= t),
// written to LDS and read back as A operands; Y = M X + (e^s C) H_in.
// ---------------------------------------------------------------------------
template <typename T, bool VEC>
__device__ __forceinline__ void head_out_body(const HeadParams& p, const HeadTile& q, float* lds) {
    const int P = p.P, N = p.N, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const HeadLds o = head_lds(P, N, true);
    float *dl = lds + o.dl, *s = lds + o.s, *w = lds + o.w, *sx = lds + o.sx, *sB = lds + o.sB, *sC = lds + o.sC;
    float* sH = lds + o.sH;   // H_in as [p][n]
    const int ldn = ld_rows_i(N);
    // entering state: from the checkpoints (rows of nchunks * N) or the chained state buffer
    const int64_t row0 = (int64_t)q.b * p.H * P + (int64_t)q.hh * P;
    const TileSrc<float> th =
        p.ckpt ? TileSrc<float>{p.ckpt + (row0 * p.nchunks + q.c) * N, (int64_t)p.nchunks * N, P, N, P, N}
               : TileSrc<float>{p.state + (((size_t)q.b * p.H + q.hh) * p.nchunks + q.c) * (size_t)N * P, N, P, N, P, N};
    float vh[16];
    tile_fetch<float, VEC>(th, vh, threadIdx.x);
    {
        HeadRegs<T> st;
        head_fetch<T, VEC>(p, q, true, st);
        tile_put<float, VEC>(th, vh, sH, ldn, false, threadIdx.x);
        head_put<T, VEC>(p, q, st, dl, s, w, sx, sB, sC, ldn, false);
    }
    // row block of this wave, rotated with the chunk so that the causal work (row block rb
    // needs columns u < 16 (rb + 1) only) spreads evenly over the SIMDs
    const int rb = (wave + q.c) & 3, t0 = 16 * rb;
    if (t0 >= q.nval) return;   // whole waves past the end (no barrier follows)
    // G rows t0.., column tiles jt <= rb, K = N.  k-group j of every MFMA takes
    // n = 16 nb + 4 j .. 16 nb + 4 j + 3 in turn, so a lane reads 4 consecutive states of a row.
    const int i = lane & 15, j = lane >> 4;
    f4 g[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) g[jt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int nb = 0; nb < N / 16; ++nb) {
        const float4 c4 = *(const float4*)&sC[(t0 + i) * ldn + 16 * nb + 4 * j];   // A[t][n] = C[t][n]
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (jt > rb) break;   // uniform
            const float4 b4 = *(const float4*)&sB[(16 * jt + i) * ldn + 16 * nb + 4 * j];   // B[n][u] = B[u][n]
            g[jt] = mfma4(c4.x, b4.x, g[jt]);
            g[jt] = mfma4(c4.y, b4.y, g[jt]);
            g[jt] = mfma4(c4.z, b4.z, g[jt]);
            g[jt] = mfma4(c4.w, b4.w, g[jt]);
        }
    }
    // mask, decay and delta: register r of lane l holds t = t0 + 4 (l/16) + r, u = 16 jt + l % 16
    float* Mw = lds + o.sM + wave * 16 * kXLd;   // this wave's rows of M
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        if (jt > rb) break;   // uniform; columns past the diagonal block are never read
        const int u = 16 * jt + (lane & 15);
        const float su = s[u], du = dl[u];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tr = 4 * (lane >> 4) + r, t = t0 + tr;
            const float m = u <= t ? g[jt][r] * __expf(s[t] - su) * du : 0.0f;
            Mw[tr * kXLd + u] = m;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done (lgkmcnt 0) before the reads below
    __builtin_amdgcn_wave_barrier();
    const float es = __expf(s[t0 + i]);   // e^(s_t) for the A operand rows
    const int tb = t0 + 4 * j;
    const bool vy = p.vy && q.nval == kHT;   // uniform
    const float* ma = Mw + i * kXLd + 4 * j;   // A[t][u] = M[t][u], u = 16 kb + 4 j + kk in turn
    for (int pt = 0; pt < P / 16; ++pt) {
        const int p0 = 16 * pt;
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // intra-chunk: K = 16 (rb + 1) (M is zero past the diagonal block)
        const float* xb = sx + (p0 + i) * kXLd + 4 * j;   // B[u][p] = X[u][p]
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb > rb) break;   // uniform
            const float4 a4 = *(const float4*)(ma + 16 * kb), b4 = *(const float4*)(xb + 16 * kb);
            acc = mfma4(a4.x, b4.x, acc);
            acc = mfma4(a4.y, b4.y, acc);
            acc = mfma4(a4.z, b4.z, acc);
            acc = mfma4(a4.w, b4.w, acc);
        }
        // carried state: K = N, n = 16 nb + 4 j + kk
        for (int nb = 0; nb < N / 16; ++nb) {
            const float4 c4 = *(const float4*)&sC[(t0 + i) * ldn + 16 * nb + 4 * j];   // e^(s_t) C[t][n]
            const float4 h4 = *(const float4*)&sH[(p0 + i) * ldn + 16 * nb + 4 * j];   // B[n][p] = H_in[p][n]
            acc = mfma4(c4.x * es, h4.x, acc);
            acc = mfma4(c4.y * es, h4.y, acc);
            acc = mfma4(c4.z * es, h4.z, acc);
            acc = mfma4(c4.w * es, h4.w, acc);
        }
        // D[t][p]: lane l, register r: t = tb + r, p = p0 + l % 16
        const int pp = p0 + i;
        T* yrow = (T*)p.y + (int64_t)q.b * p.sy[0] + ((int64_t)q.hh * P + pp) * p.sy[1] + q.t0 + tb;
        if (vy) {   // four consecutive steps in one store
            if constexpr (sizeof(T) == 2) {
                const uint32_t lo = (uint32_t)from_f32<T>(acc[0]) | ((uint32_t)from_f32<T>(acc[1]) << 16);
                const uint32_t hi = (uint32_t)from_f32<T>(acc[2]) | ((uint32_t)from_f32<T>(acc[3]) << 16);
                *(uint2*)yrow = make_uint2(lo, hi);
            } else {
                *(float4*)yrow = make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (tb + r < q.nval) yrow[r] = from_f32<T>(acc[r]);
        }
    }
}
template <typename T>
__global__ __launch_bounds__(256) void head_out_kernel(HeadParams p) {
    extern __shared__ __align__(16) float lds[];
    const HeadTile q = head_tile(p);
    const bool hal = p.ckpt ? ((uintptr_t)p.ckpt & 15) == 0 : true;   // entering-state rows aligned
    if (p.vx && p.vb && p.vc && hal && q.nval == kHT) head_out_body<T, true>(p, q, lds);   // uniform per block
    else head_out_body<T, false>(p, q, lds);
}


// ---------------------------------------------------------------------------
// Backward: the exact adjoint of the three products.  With dY the chunk's rows
// of gy, H_in its entering state and G_out the adjoint of its end state (from
// the later chunks; gh_last for the last one), the adjoint of the state at step
// u of the chunk is
//   Lam_u = sum_{t >= u} e^(s_t - s_u) C_t dY_t^T + e^(s_{T-1} - s_u) G_out,
// so that, with G = C B^T, K = dY X^T (T x T), Lm the causal decay mask,
// Mf = G o Lm, Kd = K o Lm diag(delta), e^s and ed = e^(s_{T-1} - s) per step:
//   gx = diag(delta) Z,  Z = Mf^T dY + diag(ed) B G_out,
//   gB = Kd^T C + diag(delta ed) X G_out^T,      (this head's term)
//   gC = diag(e^s) dY H_in^T + Kd B,             (this head's term)
//   gdelta_u = sum_p X[u][p] Z[u][p] + A xi_u,   gA = sum_u delta_u xi_u,
// where xi_u = sum_{t >= u} ds_t is the adjoint of log a_u and ds_t that of
// s_t: ds_t = sum_u W[t][u] - sum_v W[v][t] + e^(s_t) C_t . (dY H_in^T)_t - V_t
// (+ e^(s_{T-1}) <G_out, H_in> + sum_v V_v at t = T-1), with W = Kd o G and
// V_u = delta_u ed_u B_u . (X G_out^T)_u.  The chunk adjoints come from the
// state pass run on (gy, C) with weights e^(s_u), Q_c = C^T diag(e^s) dY, and a
// reverse chain G_out(c-1) = Q_c + e^(s_{T-1}) G_out(c); gh0 = Q_0 + decay_0 G_out(0).
// ---------------------------------------------------------------------------

// reverse chain: one thread per (batch, head, p, n), chunks from the last
// down; Q_c in gstate is replaced by G_out(c)
__global__ __launch_bounds__(256) void head_rchain_kernel(HeadBwdParams p) {
    const int P = p.P, N = p.N, NP = N * P, nch = p.nchunks;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)p.B * p.H * NP) return;
    const int64_t bh = i / NP;
    const int e = (int)(i - bh * NP), pp = e / N, n = e - pp * N;
    const int b = (int)(bh / p.H), hh = (int)(bh - (int64_t)b * p.H);
    const int64_t seq = (int64_t)b * p.H * P + (int64_t)hh * P + pp;
    float g = p.gh_last ? p.gh_last[seq * N + n] : 0.0f;
    float* S = p.gstate + (size_t)bh * nch * NP + e;
    const float* dec = p.decay + (size_t)bh * nch;
    for (int c1 = nch; c1 > 0; c1 -= kChainGroup) {
        const int c0 = max(0, c1 - kChainGroup);
        float loc[kChainGroup], dc[kChainGroup];
#pragma unroll
        for (int j = 0; j < kChainGroup; ++j)
            if (c0 + j < c1) {
                loc[j] = S[(size_t)(c0 + j) * NP];
                dc[j] = dec[c0 + j];
            }
#pragma unroll
        for (int j = kChainGroup - 1; j >= 0; --j)
            if (c0 + j < c1) {
                S[(size_t)(c0 + j) * NP] = g;
                g = fmaf(dc[j], g, loc[j]);
            }
    }
    if (p.gh0) p.gh0[seq * N + n] = g;
}

// Mf and Kd are kept transposed, as [u][t], for t >= u's 16-row block only:
// row u of block ub = u / 16 holds t = 16 ub .. T-1 (64 - 16 ub values) with
// 4 floats of padding, so the rows of a block start 4 or 20 banks apart.
__host__ __device__ constexpr int ct_ld(int ub) { return kHT - 16 * ub + 4; }
__host__ __device__ constexpr int ct_off(int ub) { return 16 * ((kHT + 4) * ub - 8 * ub * (ub - 1)); }
constexpr int kCtSize = ct_off(4);   // 2816 floats

// LDS layout (float offsets, multiples of 4): delta and s (T each); the W row
// sums per 16-column block and column sums per 16-row block (4 x T each),
// sum_p X Z per 16-channel block (4 x T), the carried term minus V (T), and
// misc = <G_out, H_in> and the four 16-step block sums of V; x and gy as
// [p][t], B and C as [t][n], H_in and G_out as [p][n]; Mf and Kd in the causal
// layout above.  At P = 64, N = 16 this is 81696 bytes: two workgroups per CU.
struct HeadBwdLds {
    int dl, s, wrow, wcol, expl, cv, misc, sx, sy, sB, sC, sH, sG, MT, KT, total;
};
__host__ __device__ inline HeadBwdLds head_bwd_lds(int P, int N) {
    const int ldn = ld_rows_i(N);
    HeadBwdLds o;
    o.dl = 0;
    o.s = kHT;
    o.wrow = 2 * kHT;
    o.wcol = o.wrow + 4 * kHT;   // follows wrow: the two are cleared as one run of 8 T
    o.expl = o.wcol + 4 * kHT;
    o.cv = o.expl + 4 * kHT;
    o.misc = o.cv + kHT;
    o.sx = o.misc + 8;
    o.sy = o.sx + P * kXLd;
    o.sB = o.sy + P * kXLd;
    o.sC = o.sB + kHT * ldn;
    o.sH = o.sC + kHT * ldn;
    o.sG = o.sH + P * ldn;
    o.MT = o.sG + P * ldn;
    o.KT = o.MT + kCtSize;
    o.total = o.KT + kCtSize;
    return o;
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations complete,
// then s_barrier (a plain __syncthreads would first wait for the gx and partial
// sum stores in flight as well).
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr int kBwdThreads = 512;

// sum over the 64 lanes, the same value in every lane
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) v += __shfl_xor(v, k);
    return v;
}

template <typename T, bool VEC>
__device__ __forceinline__ void head_bwd_body(const HeadBwdParams& p, const HeadTile& q, float* lds) {
    const int P = p.P, N = p.N, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ldn = ld_rows_i(N), i = lane & 15, j = lane >> 4;
    const HeadBwdLds o = head_bwd_lds(P, N);
    float *dl = lds + o.dl, *s = lds + o.s;
    float *wrow = lds + o.wrow, *wcol = lds + o.wcol, *expl = lds + o.expl, *cv = lds + o.cv;
    float *misc = lds + o.misc, *sx = lds + o.sx, *sy = lds + o.sy, *sB = lds + o.sB;
    float *sC = lds + o.sC, *sH = lds + o.sH, *sG = lds + o.sG, *MT = lds + o.MT, *KT = lds + o.KT;
    const int64_t bh = (int64_t)q.b * p.H + q.hh;
    const int64_t row0 = bh * P;   // channel row (b, h*P) of the (B, D, ...) arrays
    const float A = p.A[(int64_t)q.hh * p.sA];

    // loads: threads 0-255 take x, B and H_in, threads 256-511 gy, C and G_out (uniform per wave)
    {
        const int grp = tid >> 8, gt = tid & 255;
        const TileSrc<T> t0s =
            grp ? TileSrc<T>{(const T*)p.gy + (int64_t)q.b * p.sgy[0] + (int64_t)q.hh * P * p.sgy[1] + q.t0,
                             p.sgy[1], P, kHT, P, q.nval}
                : TileSrc<T>{(const T*)p.x + (int64_t)q.b * p.sx[0] + (int64_t)q.hh * P * p.sx[1] + q.t0, p.sx[1], P,
                             kHT, P, q.nval};
        const TileSrc<T> t1s =
            grp ? TileSrc<T>{(const T*)p.C + (int64_t)q.b * p.sC[0] + (int64_t)q.t0 * p.sC[2], p.sC[2], kHT, N,
                             q.nval, N}
                : TileSrc<T>{(const T*)p.Bm + (int64_t)q.b * p.sBm[0] + (int64_t)q.t0 * p.sBm[2], p.sBm[2], kHT, N,
                             q.nval, N};
        const TileSrc<float> t2s =
            grp ? TileSrc<float>{p.gstate + ((size_t)bh * p.nchunks + q.c) * (size_t)N * P, N, P, N, P, N}
                : TileSrc<float>{p.ckpt + (row0 * p.nchunks + q.c) * N, (int64_t)p.nchunks * N, P, N, P, N};
        float v0[16], v1[16], v2[16];
        tile_fetch<T, VEC>(t0s, v0, gt);
        tile_fetch<T, VEC>(t1s, v1, gt);
        tile_fetch<float, VEC>(t2s, v2, gt);
        float dv = 0.0f;
        if (tid < kHT) {
            const T* delta = (const T*)p.delta + (int64_t)q.b * p.sdelta[0] + (int64_t)q.hh * p.sdelta[1] + q.t0;
            dv = tid < q.nval ? to_f32(delta[min(tid, q.nval - 1)]) : 0.0f;
        }
        wrow[tid] = 0.0f;   // wrow and wcol: 8 T = 512 floats
        tile_put<T, VEC>(t0s, v0, grp ? sy : sx, kXLd, false, gt);
        tile_put<T, VEC>(t1s, v1, grp ? sC : sB, ldn, false, gt);
        tile_put<float, VEC>(t2s, v2, grp ? sG : sH, ldn, false, gt);
        if (tid < kHT) {   // wave 0, lane = step: s = A * inclusive prefix sum of delta
            float v = dv;
            v += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, v);
            const float r0 = __shfl(v, 15), r1 = __shfl(v, 31), r2 = __shfl(v, 47);
            const int row = tid >> 4;
            v += (row > 0 ? r0 : 0.0f) + (row > 1 ? r1 : 0.0f) + (row > 2 ? r2 : 0.0f);
            dl[tid] = dv;
            s[tid] = A * v;
        }
    }
    __syncthreads();

    // phase 1: the ten causal 16 x 16 blocks (tb >= ub) of G and K, masked and scaled in registers
    // into Mf and Kd (stored transposed), and the row and column sums of W = Kd o G
    for (int idx = wave; idx < 10; idx += kBwdThreads / 64) {   // uniform per wave
        const int tb = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3, ub = idx - tb * (tb + 1) / 2;
        const int t0 = 16 * tb, u0 = 16 * ub;
        f4 ga = {0.0f, 0.0f, 0.0f, 0.0f}, ka = {0.0f, 0.0f, 0.0f, 0.0f};
        // G[t][u] = sum_n C[t][n] B[u][n]; k-group j takes n = 16 nb + 4 j .. + 3 in turn
        for (int nb = 0; nb < N / 16; ++nb) {
            const float4 c4 = *(const float4*)&sC[(t0 + i) * ldn + 16 * nb + 4 * j];
            const float4 b4 = *(const float4*)&sB[(u0 + i) * ldn + 16 * nb + 4 * j];
            ga = mfma4(c4.x, b4.x, ga);
            ga = mfma4(c4.y, b4.y, ga);
            ga = mfma4(c4.z, b4.z, ga);
            ga = mfma4(c4.w, b4.w, ga);
        }
        // K[t][u] = sum_p dY[t][p] X[u][p]: A[t][p] = sy[p][t], B[p][u] = sx[p][u], k-group j = p % 4
        for (int p16 = 0; p16 < P / 16; ++p16)
#pragma unroll
        for (int p4 = 4 * p16; p4 < 4 * p16 + 4; ++p4) {
            const int pr = 4 * p4 + j;
            ka = mfma4(sy[pr * kXLd + t0 + i], sx[pr * kXLd + u0 + i], ka);
        }
        // register r of lane l: t = t0 + 4 j + r, u = u0 + i
        const int u = u0 + i;
        const float su = s[u], du = dl[u];
        f4 mf, kd;
        float rs[4], cs = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + 4 * j + r;
            const float e = u <= t ? __expf(s[t] - su) : 0.0f;
            mf[r] = ga[r] * e;
            kd[r] = ka[r] * e * du;
            rs[r] = kd[r] * ga[r];
            cs += rs[r];
        }
        const int ca = ct_off(ub) + i * ct_ld(ub) + 16 * (tb - ub) + 4 * j;   // (u, t0 + 4 j)
        *(f4*)&MT[ca] = mf;
        *(f4*)&KT[ca] = kd;
#pragma unroll
        for (int r = 0; r < 4; ++r) {   // sum over the 16 lanes of each row: the total lands in lane 15
            float v = rs[r];
            v += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, v);
            v += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, v);
            rs[r] = v;
        }
        if (i == 15) *(float4*)&wrow[ub * kHT + t0 + 4 * j] = make_float4(rs[0], rs[1], rs[2], rs[3]);
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        if (j == 0) wcol[tb * kHT + u] = cs;
    }
    if (wave == kBwdThreads / 64 - 1) {   // <G_out, H_in>
        float v = 0.0f;
        for (int e = lane; e < P * N; e += 64) {
            const int pp = e / N, n = e - pp * N;
            v += sG[pp * ldn + n] * sH[pp * ldn + n];
        }
        v = wave_sum(v);
        if (lane == 0) misc[0] = v;
    }
    lds_barrier();

    // phase 2.  Waves 0-3: gB for steps 16w.. and gC for steps 16w.. (per-head terms, [n][t]).
    // Waves 4-7: Z for channels 16(w-4).. and every step: gx and sum_p X Z.
    const int64_t pofs = ((int64_t)q.hh * p.B + q.b) * N * (int64_t)p.L + q.t0;
    const float sT = s[kHT - 1];
    if (wave < 4) {
        const int b0 = 16 * wave;
        const float* kb = KT + ct_off(wave) + i * ct_ld(wave) - b0;   // row u = b0 + i of Kd^T, by t
        float vsum = 0.0f, csum = 0.0f;
        for (int nt = 0; nt < N / 16; ++nt) {
            f4 a1 = {0.0f, 0.0f, 0.0f, 0.0f}, a2 = {0.0f, 0.0f, 0.0f, 0.0f};
            // Kd^T C over the row blocks tb >= this block: A[n][t] = C[t][n], B[t][u] = KT[u][t]
            for (int tb = wave; tb < 4; ++tb) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int t = 16 * tb + 4 * kk + j;
                    a1 = mfma4(sC[t * ldn + 16 * nt + i], kb[t], a1);
                }
            }
            // X G_out^T: A[n][p] = G_out[p][n], B[p][u] = sx[p][u]
            for (int p16 = 0; p16 < P / 16; ++p16)
#pragma unroll
            for (int p4 = 4 * p16; p4 < 4 * p16 + 4; ++p4) {
                const int pr = 4 * p4 + j;
                a2 = mfma4(sG[pr * ldn + 16 * nt + i], sx[pr * kXLd + b0 + i], a2);
            }
            // register r of lane l: n = 16 nt + 4 j + r, u = b0 + i
            {
                const int u = b0 + i;
                const float sc = dl[u] * __expf(sT - s[u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = 16 * nt + 4 * j + r;
                    const float b2 = sc * a2[r];
                    vsum += sB[u * ldn + n] * b2;
                    if (p.partB && u < q.nval) p.partB[pofs + (int64_t)n * p.L + u] = a1[r] + b2;
                }
            }
            f4 c1 = {0.0f, 0.0f, 0.0f, 0.0f}, c2 = {0.0f, 0.0f, 0.0f, 0.0f};
            // dY H_in^T: A[n][p] = H_in[p][n], B[p][t] = sy[p][t]
            for (int p16 = 0; p16 < P / 16; ++p16)
#pragma unroll
            for (int p4 = 4 * p16; p4 < 4 * p16 + 4; ++p4) {
                const int pr = 4 * p4 + j;
                c1 = mfma4(sH[pr * ldn + 16 * nt + i], sy[pr * kXLd + b0 + i], c1);
            }
            // Kd B over the column blocks ub <= this block: A[n][u] = B[u][n], B[u][t] = KT[u][t]
            for (int ub = 0; ub <= wave; ++ub) {
                const float* kc = KT + ct_off(ub) + b0 - 16 * ub + i;   // column t = b0 + i of Kd^T
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int u = 16 * ub + 4 * kk + j;
                    c2 = mfma4(sB[u * ldn + 16 * nt + i], kc[(4 * kk + j) * ct_ld(ub)], c2);
                }
            }
            // register r of lane l: n = 16 nt + 4 j + r, t = b0 + i
            {
                const int t = b0 + i;
                const float e = __expf(s[t]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = 16 * nt + 4 * j + r;
                    const float g1 = e * c1[r];
                    csum += sC[t * ldn + n] * g1;
                    if (p.partC && t < q.nval) p.partC[pofs + (int64_t)n * p.L + t] = g1 + c2[r];
                }
            }
        }
        vsum += __shfl_xor(vsum, 16);
        vsum += __shfl_xor(vsum, 32);
        csum += __shfl_xor(csum, 16);
        csum += __shfl_xor(csum, 32);
        if (j == 0) cv[b0 + i] = csum - vsum;
        // this block's total of V: lane 15 of the first row ends with it
        vsum += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, vsum);
        vsum += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, vsum);
        vsum += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, vsum);
        vsum += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, vsum);
        if (lane == 15) misc[1 + wave] = vsum;
    } else if (16 * (wave - 4) < P) {
        const int pt = wave - 4, p0 = 16 * pt;
        T* gx = (T*)p.gx;
        T* gxrow = gx ? gx + (int64_t)q.b * p.sgx[0] + ((int64_t)q.hh * P + p0 + i) * p.sgx[1] + q.t0 : nullptr;
        const bool vgx = p.vgx && q.nval == kHT;   // uniform: four steps in one store
        for (int ub = 0; ub < 4; ++ub) {
            const int u0 = 16 * ub;
            f4 z1 = {0.0f, 0.0f, 0.0f, 0.0f}, z2 = {0.0f, 0.0f, 0.0f, 0.0f};
            // Mf^T dY (Z[u][p] = sum_t Mf[t][u] dY[t][p]) over the row blocks tb >= ub;
            // k-group j takes t = 16 tb + 4 j .. + 3 in turn
            for (int tb = ub; tb < 4; ++tb) {
                const float4 a4 = *(const float4*)&MT[ct_off(ub) + i * ct_ld(ub) + 16 * (tb - ub) + 4 * j];
                const float4 b4 = *(const float4*)&sy[(p0 + i) * kXLd + 16 * tb + 4 * j];
                z1 = mfma4(a4.x, b4.x, z1);
                z1 = mfma4(a4.y, b4.y, z1);
                z1 = mfma4(a4.z, b4.z, z1);
                z1 = mfma4(a4.w, b4.w, z1);
            }
            // B G_out (Z[u][p] = sum_n B[u][n] G_out[p][n])
            for (int nb = 0; nb < N / 16; ++nb) {
                const float4 a4 = *(const float4*)&sB[(u0 + i) * ldn + 16 * nb + 4 * j];
                const float4 b4 = *(const float4*)&sG[(p0 + i) * ldn + 16 * nb + 4 * j];
                z2 = mfma4(a4.x, b4.x, z2);
                z2 = mfma4(a4.y, b4.y, z2);
                z2 = mfma4(a4.z, b4.z, z2);
                z2 = mfma4(a4.w, b4.w, z2);
            }
            // register r of lane l: u = u0 + 4 j + r, p = p0 + i
            const int ua = u0 + 4 * j;
            const float4 x4 = *(const float4*)&sx[(p0 + i) * kXLd + ua];
            const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
            float g[4], ex[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = z1[r] + __expf(sT - s[ua + r]) * z2[r];
                g[r] = dl[ua + r] * z;
                ex[r] = xs[r] * z;
            }
            if (vgx) {
                if constexpr (sizeof(T) == 2) {
                    const uint32_t lo = (uint32_t)from_f32<T>(g[0]) | ((uint32_t)from_f32<T>(g[1]) << 16);
                    const uint32_t hi = (uint32_t)from_f32<T>(g[2]) | ((uint32_t)from_f32<T>(g[3]) << 16);
                    *(uint2*)(gxrow + ua) = make_uint2(lo, hi);
                } else {
                    *(float4*)(gxrow + ua) = make_float4(g[0], g[1], g[2], g[3]);
                }
            } else if (gxrow) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ua + r < q.nval) gxrow[ua + r] = from_f32<T>(g[r]);
            }
            // sum over the 16 channels of each row of lanes: lane 15 of row j ends with steps ua .. ua + 3
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = ex[r];
                v += dpp<SSM_DPP_ROW_SHR(1)>(0.0f, v);
                v += dpp<SSM_DPP_ROW_SHR(2)>(0.0f, v);
                v += dpp<SSM_DPP_ROW_SHR(4)>(0.0f, v);
                v += dpp<SSM_DPP_ROW_SHR(8)>(0.0f, v);
                ex[r] = v;
            }
            if (i == 15) *(float4*)&expl[pt * kHT + ua] = make_float4(ex[0], ex[1], ex[2], ex[3]);
        }
    }
    lds_barrier();

    // phase 3 (wave 0, lane = step): ds, its suffix sums xi, gdelta and this chunk's term of gA
    if (wave == 0) {
        const int u = lane;
        const float rw = ((wrow[u] + wrow[kHT + u]) + wrow[2 * kHT + u]) + wrow[3 * kHT + u];
        const float cw = ((wcol[u] + wcol[kHT + u]) + wcol[2 * kHT + u]) + wcol[3 * kHT + u];
        float ds = rw - cw + cv[u];
        if (u == kHT - 1) ds += __expf(sT) * misc[0] + (((misc[1] + misc[2]) + misc[3]) + misc[4]);
        float xi = ds;
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) {
            const float y = __shfl_down(xi, k);
            if (u + k < 64) xi += y;
        }
        float ex = 0.0f;
        for (int pt = 0; pt < P / 16; ++pt) ex += expl[pt * kHT + u];
        if (p.gdelta && u < q.nval)
            ((T*)p.gdelta)[(int64_t)q.b * p.sgdelta[0] + (int64_t)q.hh * p.sgdelta[1] + q.t0 + u] =
                from_f32<T>(ex + A * xi);
        const float ga = wave_sum(dl[u] * xi);
        if (p.partA && u == 0) p.partA[((int64_t)q.hh * p.B + q.b) * p.nchunks + q.c] = ga;
    }
}
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void head_bwd_kernel(HeadBwdParams p) {
    extern __shared__ __align__(16) float lds[];
    const HeadTile q = head_tile(p);
    const bool hal = ((uintptr_t)p.ckpt & 15) == 0;
    if (p.vx && p.vgy && p.vb && p.vc && hal && q.nval == kHT) head_bwd_body<T, true>(p, q, lds);   // uniform
    else head_bwd_body<T, false>(p, q, lds);
}


// out[h] = part[h * n] + ... + part[h * n + n - 1], in order (gA from its per-(batch, chunk) terms)
__global__ __launch_bounds__(64) void head_sum_rows_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                           int H, int n) {
    const int hh = blockIdx.x * 64 + threadIdx.x;
    if (hh >= H) return;
    float acc = 0.0f;
    for (int e = 0; e < n; ++e) acc += part[(int64_t)hh * n + e];
    out[hh] = acc;
}

hipError_t launch_head_state(const HeadParams& p, int dtype, hipStream_t st) {
    if (p.P % 16 || p.P > 64 || p.N % 16 || p.N > 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.nchunks, (unsigned)p.H, (unsigned)p.B);
    const size_t lds = head_lds(p.P, p.N, false).total * sizeof(float);
    if (dtype == 0) head_state_kernel<float><<<grid, 256, lds, st>>>(p);
    else head_state_kernel<bf16_t><<<grid, 256, lds, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_chain(const HeadParams& p, hipStream_t st) {
    const int64_t n = (int64_t)p.B * p.H * p.N * p.P;
    head_chain_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_out(const HeadParams& p, int dtype, hipStream_t st) {
    if (p.P % 16 || p.P > 64 || p.N % 16 || p.N > 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.nchunks, (unsigned)p.H, (unsigned)p.B);
    const size_t lds = head_lds(p.P, p.N, true).total * sizeof(float);
    if (dtype == 0) head_out_kernel<float><<<grid, 256, lds, st>>>(p);
    else head_out_kernel<bf16_t><<<grid, 256, lds, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_rchain(const HeadBwdParams& p, hipStream_t st) {
    const int64_t n = (int64_t)p.B * p.H * p.N * p.P;
    head_rchain_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_bwd(const HeadBwdParams& p, int dtype, hipStream_t st) {
    if (p.P % 16 || p.P > 64 || p.N % 16 || p.N > 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.nchunks, (unsigned)p.H, (unsigned)p.B);
    const size_t lds = head_bwd_lds(p.P, p.N).total * sizeof(float);
    if (dtype == 0) head_bwd_kernel<float><<<grid, kBwdThreads, lds, st>>>(p);
    else head_bwd_kernel<bf16_t><<<grid, kBwdThreads, lds, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_head_sum_rows(const float* part, float* out, int H, int n, hipStream_t st) {
    head_sum_rows_kernel<<<(unsigned)((H + 63) / 64), 64, 0, st>>>(part, out, H, n);
    return hipGetLastError();
}

}  // namespace ssm
