// Diagonal real scan with the transition diagonal a_t and input term b_t given
// as (B,D,L,N) tensors (the generic h_t = a_t h_{t-1} + b_t, y_t = C_t . h_t).
//
// Work mapping.  This mode streams 8 bytes per element and does one fma, so it
// is bound by HBM, not by arithmetic: a 16-lane row holds the N states of one
// (batch, channel) and walks time sequentially, so every step of a row moves
// one contiguous 64-byte line of a and of b.  y_t = sum_n C_t[n] h_t[n] is kept
// per step for 16 steps and summed across the row with one transpose-reduction.
// Segments of 32-step chunks along L run in parallel (summary / combine /
// re-run, as for the other modes).  The backward recomputes each 32-step chunk
// from its checkpoint into registers and runs the adjoint nu_t = a_t lambda_t
// backwards; sums over channels (gC) are taken over the 16 rows in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kDChunk = 32;

// Steps tb .. tb+K-1 of state n of a (L,N) row-major stream.  When the whole
// block lies inside the sequence the loads are unconditional, so all K are in
// flight together; otherwise steps past L read `fill`.
template <int K>
__device__ __forceinline__ void load_steps(const float* __restrict__ row, int tb, int L, int N, int n, float fill,
                                           float (&v)[K]) {
    const float* __restrict__ q = row + (size_t)tb * N + n;   // step j at q[j * N]: immediate offsets when N is fixed
    if (tb + K <= L) {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = q[j * N];
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = (tb + j < L) ? q[j * N] : fill;
    }
}

// Forward.  Time is walked in 16-step blocks; the a and b values of the next
// block are loaded while the current block is computed (two register sets),
// and C of the current block is requested before them.
template <bool SUMMARY, int NT>
__global__ __launch_bounds__(256) void dense_fwd_kernel(DenseParams p) {
    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;  // NT = 16: compile-time state count
    const bool nl = lane < N;
    const int n = nl ? lane : N - 1;     // lanes past N load a valid state and discard it
    const size_t seq = (size_t)b * p.D + dc;
    float h = 0.0f, P = 1.0f;
    if (!SUMMARY && nl) {
        if (p.G > 1) h = p.carry_in[(seq * p.G + g) * N + n];
        else if (p.h0) h = p.h0[seq * N + n];
    }
    const int c0 = g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const float* arow = p.a + seq * L * N;
    const float* brow = p.b + seq * L * N;
    const float* crow = p.C + (size_t)b * L * N;
    constexpr int BPC = kDChunk / 16;   // 16-step blocks per chunk
    const int k0 = c0 * BPC;
    const int k1 = min(c1 * BPC, (L + 15) / 16);

    auto block = [&](int k, const float (&av)[16], const float (&bv)[16]) {
        const int tb = 16 * k;
        if (!SUMMARY && (k % BPC) == 0 && p.ckpt_out && act && nl)
            p.ckpt_out[(seq * p.nchunks + k / BPC) * N + n] = h;
        float cv[16];
        if (!SUMMARY) load_steps<16>(crow, tb, L, N, n, 0.0f, cv);
        float yp[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const bool on = nl && tb + j < L;
            const float a = on ? av[j] : 1.0f;
            h = fmaf(a, h, on ? bv[j] : 0.0f);
            if (SUMMARY) P *= a;
            else yp[j] = on ? cv[j] * h : 0.0f;
        }
        if (!SUMMARY && p.y) {
            const float ys = row_transpose_sum16(yp);
            const int t = tb + lane;
            if (act && t < L) p.y[seq * L + t] = ys;
        }
    };

    float a0[16], b0[16], a1[16], b1[16];
    if (k0 < k1) {
        load_steps<16>(arow, 16 * k0, L, N, n, 1.0f, a0);
        load_steps<16>(brow, 16 * k0, L, N, n, 0.0f, b0);
    }
    for (int k = k0; k < k1; k += 2) {
        if (k + 1 < k1) {
            load_steps<16>(arow, 16 * (k + 1), L, N, n, 1.0f, a1);
            load_steps<16>(brow, 16 * (k + 1), L, N, n, 0.0f, b1);
        }
        block(k, a0, b0);
        if (k + 1 >= k1) break;
        if (k + 2 < k1) {
            load_steps<16>(arow, 16 * (k + 2), L, N, n, 1.0f, a0);
            load_steps<16>(brow, 16 * (k + 2), L, N, n, 0.0f, b0);
        }
        block(k + 1, a1, b1);
    }
    if (!act || !nl) return;
    if (SUMMARY) {
        p.segP[(seq * p.G + g) * N + n] = P;
        p.segS[(seq * p.G + g) * N + n] = h;
    } else if (p.h_last && g == p.G - 1) {
        p.h_last[seq * N + n] = h;
    }
}

// gC partials of one chunk: [row][step][state] with rows padded by 16 floats
constexpr int kDRedRow = kDChunk * 16 + 16;

// Backward, reverse over chunks.  Per chunk every load (checkpoint, gy, a, b,
// C) is issued before any use; the chunk's states are recomputed into
// registers, then the adjoint runs right to left.
template <bool SUMMARY, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void dense_bwd_kernel(DenseParams p) {
    __shared__ float red[SUMMARY ? 4 : 16 * kDRedRow];
    const int tid = threadIdx.x, lane = tid & 15, row = tid >> 4;
    const int b = blockIdx.y, g = blockIdx.z;
    const int d = blockIdx.x * 16 + row;
    const bool act = d < p.D;
    const int dc = act ? d : p.D - 1;
    const int N = NT ? NT : p.N, L = p.L;  // NT = 16: compile-time state count
    const bool nl = lane < N;
    const int n = nl ? lane : N - 1;
    const size_t seq = (size_t)b * p.D + dc;
    float nu = 0.0f, Q = 1.0f;
    if (!SUMMARY && nl) {
        if (p.G > 1) nu = p.nu_in[(seq * p.G + g) * N + n];
        else if (p.gh_last) nu = p.gh_last[seq * N + n];
    }
    const int c0 = g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const float* arow = p.a + seq * L * N;
    const float* brow = p.b + seq * L * N;
    const float* crow = p.C + (size_t)b * L * N;
    const float live = act ? 1.0f : 0.0f;
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const int t0 = ch * kDChunk;
        // gy of the chunk: lane l holds steps l and l + 16
        float gyl[kDChunk / 16];
#pragma unroll
        for (int q = 0; q < kDChunk / 16; ++q) {
            const int t = t0 + 16 * q + lane;
            gyl[q] = t < L ? p.gy[seq * L + t] * live : 0.0f;
        }
        float as[kDChunk], cs[kDChunk];
        load_steps<kDChunk>(arow, t0, L, N, n, 1.0f, as);
        load_steps<kDChunk>(crow, t0, L, N, n, 0.0f, cs);
        if (SUMMARY) {
#pragma unroll
            for (int jj = kDChunk - 1; jj >= 0; --jj) {
                const float gyt = bcast16(gyl[jj / 16], jj % 16);
                const float av = nl ? as[jj] : 1.0f;
                nu = av * fmaf(nl ? cs[jj] : 0.0f, gyt, nu);
                Q *= av;
            }
            continue;
        }
        float hs[kDChunk + 1];
        {
            float bs[kDChunk];
            load_steps<kDChunk>(brow, t0, L, N, n, 0.0f, bs);
            hs[0] = p.ckpt[(seq * p.nchunks + ch) * N + n];
#pragma unroll
            for (int j = 0; j < kDChunk; ++j) hs[j + 1] = fmaf(as[j], hs[j], bs[j]);
        }
        float* rrow = red + row * kDRedRow;
        const bool wr = act && nl;
#pragma unroll
        for (int j = kDChunk - 1; j >= 0; --j) {
            const int t = t0 + j;
            const float gyt = bcast16(gyl[j / 16], j % 16);
            const bool on = nl && t < L;
            const float lam = fmaf(cs[j], gyt, nu);
            if (wr && t < L) {
                const size_t o = (size_t)t * N + n;
                if (p.ga) p.ga[seq * L * N + o] = lam * hs[j];
                if (p.gb) p.gb[seq * L * N + o] = lam;
            }
            if (p.partC) rrow[j * 16 + lane] = on ? gyt * hs[j + 1] : 0.0f;
            nu = on ? as[j] * lam : nu;
        }
        if (p.partC) {
            __syncthreads();
            for (int o = tid; o < kDChunk * 16; o += 256) {
                const int tt = o / 16, nn = o % 16;
                float s = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) s += red[r * kDRedRow + tt * 16 + nn];
                const int t = t0 + tt;
                if (t < L && nn < N) p.partC[(((size_t)blockIdx.x * p.B + b) * N + nn) * L + t] = s;
            }
            __syncthreads();
        }
    }
    if (!act || !nl) return;
    if (SUMMARY) {
        p.segQ[(seq * p.G + g) * N + n] = Q;
        p.segR[(seq * p.G + g) * N + n] = nu;
    } else if (p.gh0 && g == 0) {
        p.gh0[seq * N + n] = nu;
    }
}

hipError_t launch_dense_fwd(const DenseParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.D + 15) / 16, p.B, p.G);
    if (p.N == 16) {
        if (summary) dense_fwd_kernel<true, 16><<<grid, 256, 0, st>>>(p);
        else dense_fwd_kernel<false, 16><<<grid, 256, 0, st>>>(p);
    } else {
        if (summary) dense_fwd_kernel<true, 0><<<grid, 256, 0, st>>>(p);
        else dense_fwd_kernel<false, 0><<<grid, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_dense_bwd(const DenseParams& p, bool summary, hipStream_t st) {
    dim3 grid((p.D + 15) / 16, p.B, p.G);
    // the backward keeps the generic state count: at N = 16 the specialised
    // variant measured slower (its register allocation spills more)
    if (summary) dense_bwd_kernel<true, 0><<<grid, 256, 0, st>>>(p);
    else dense_bwd_kernel<false, 0><<<grid, 256, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace ssm
