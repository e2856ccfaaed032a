// Internal interface between the host library (api.cpp) and the HIP kernels.
// Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

// ------------------------------- real, selective ---------------------------
// Step sizes taken from the input-projection output z: delta = softplus(z + bias[d])
// (softplus = 1) or z + bias[d]; both off: delta as given.
struct StepXform {
    const float* bias;  // (D) or null
    int softplus;
};
// Selective kernel variants: input term and where B_t, C_t come from.
constexpr int kVarEuler = 0;   // Euler input term, B_t / C_t shared by the channels (LDS tiles)
constexpr int kVarPerD = 1;    // Euler input term, B_t / C_t per channel (read by each row)
constexpr int kVarZoh = 2;     // zero-order-hold input term, B_t / C_t shared by the channels

// Strides of the selective mode's streamed views, in elements: (B,D,L)
// streams s[0] batch, s[1] channel (steps contiguous); B_t, C_t (B,D,L,N)
// s[0] batch, s[1] channel (0 = shared by the channels), s[2] step; A (D,N)
// channel stride sA.
struct SelFwdParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C;
    int64_t sdelta[2], sx[2], sy[2], sBm[3], sC[3], sA;
    int bc_vec;             // 16-byte loads of the B_t / C_t rows (aligned)
    int var;                // kernel variant: 0 Euler, 1 per-channel B_t / C_t, 2 ZOH
    // channels per delta row and per A row (one scalar transition per head of
    // dgrp = agrp channels), and A's state stride (0: one value for every state)
    int dgrp = 1, agrp = 1;
    int64_t sAn = 1;
    const float* h0;        // (B,D,N) or null
    const float* carry_in;  // (B,D,G,N) state entering each segment (G > 1)
    void* y;                // (B,D,L) or null
    float* h_last;          // (B,D,N) or null
    float* ckpt;            // (B,D,ntiles,N) or null
    float* segP;            // summary pass: product of a over each segment (B,D,G,N)
    float* segS;            // summary pass: local state at segment end (B,D,G,N)
    float* tile_dsum;       // (B,D,ntiles) sum of delta over each tile, or null
    // main pass with the impulse sensitivity (B_t, C_t shared, Euler): s = d y[t_out] / d x,
    // (B,D,L) dense, from send = (B,D,ntiles) sums of delta over later tiles up to t_out
    void* s = nullptr;
    void* s_delta = nullptr;   // with it also d y[t_out] / d delta, (B,D,L) dense
    const double* send = nullptr;
    int t_out = 0;
    StepXform stepf;
    int B, D, L, N, ntiles, tiles_per_seg, G, vec;
};
struct SelBwdParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C;
    const void* gy; const float* gh_last; const float* ckpt;
    int64_t sdelta[2], sx[2], sgy[2], sgx[2], sgdelta[2], sBm[3], sC[3], sA;
    int bc_vec;
    int var;
    int dgrp = 1, agrp = 1;
    int64_t sAn = 1;
    int gdelta_f32 = 0;     // gdelta stored as fp32 whatever the stream type
    void* gBm_pd; void* gC_pd;   // per-channel B_t, C_t: their gradients (B,D,L,N), written directly
    const float* nu_in;     // (B,D,G,N) adjoint entering each segment from the right (G > 1)
    void* gdelta; void* gx; float* gh0;
    float* partB; float* partC;  // (nblk,B,N,L) partial sums over each block of channels
    float* partA;                // (B,G,D,N)
    float* partBias;             // (B,G,D) partial sums of the step-size bias gradient, or null
    float* segQ; float* segR;    // summary pass outputs (B,D,G,N)
    StepXform stepf;
    int B, D, L, N, ntiles, tiles_per_seg, G, vec;
    // checkpoints of tile k at index k * ckpt_every of ckpt_tiles per sequence (0: ntiles, 1)
    int ckpt_tiles = 0, ckpt_every = 1;
};
struct SensParams {
    const void* delta; const float* A; const void* Bm; const void* C;
    int64_t sdelta[2], sx[2], sBm[3], sC[3], sA;   // views, as in SelFwdParams (B_t, C_t shared)
    const double* send;     // (B,D,ntiles) sum of delta over later steps up to t_out
    void* s;                // nullable d y[t_out] / d x
    const void* x; const float* ckpt;   // with s_delta: inputs and the states entering each tile
    void* s_delta;          // nullable d y[t_out] / d delta
    StepXform stepf;
    int B, D, L, N, ntiles, t_out, vec;
    int tiles_per_wg;       // set by the launcher: grid.z stays within its limit for any L
};

// Rows r = 0..R-1 of the input Jacobian, s[r] = d y[t0 + r] / d x (R <= kSensRowsMax).
constexpr int kSensRowsMax = 16;
struct SensRowsParams {
    const void* delta; const float* A; const void* Bm; const void* C;
    int64_t sdelta[2], sBm[3], sC[3], sA;
    int bc_vec;
    const double* send;     // (B,D,ntiles) sum of delta over later steps up to t0 (64-step tiles)
    float* w;               // (B,D,R,N) C_{t0+r}[n] * prod_{t0 < s <= t0+r} a_s[n]
    void* s;                // (R,B,D,L)
    StepXform stepf;
    int B, D, L, N, ntiles, t0, R, vec;
    int tiles_per_wg;       // set by the launcher: grid.z stays within its limit for any L
};

// dst[0..n) = src (or 0 when src is NULL); nothing when dst is NULL or n is 0
hipError_t launch_fill_copy_f32(float* dst, const float* src, size_t n, hipStream_t st);
hipError_t launch_zero_bytes(void* dst, size_t bytes, hipStream_t st);  // bytes even

hipError_t launch_sel_fwd(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
hipError_t launch_sel_bwd(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
// the variants (selective_perd.hip, selective_zoh.hip)
hipError_t launch_sel_fwd_perd(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
hipError_t launch_sel_bwd_perd(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
hipError_t launch_sel_fwd_zoh(const SelFwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
// main forward pass that also forms the impulse sensitivity, and with s_delta the step-size sensitivity
// (selective_sens.hip; N = 16, Euler, shared B_t, C_t)
hipError_t launch_sel_fwd_sens(const SelFwdParams& p, int dtype, int kpl, hipStream_t st);
hipError_t launch_sel_bwd_zoh(const SelBwdParams& p, int dtype, int kpl, bool summary, hipStream_t st);
int sel_bwd_rows();  // channels per backward workgroup (one gB/gC partial per block)
hipError_t launch_seg_combine_fwd(const float* P, const float* S, const float* h0, float* carry_in,
                                  int BD, int G, int N, hipStream_t st);
hipError_t launch_seg_combine_rev(const float* Q, const float* R, const float* nu_last, float* nu_in,
                                  int BD, int G, int N, hipStream_t st);
// (nblk, B, N, L) channel-block partials of gB and/or gC (null skips) -> (B, L, N)
hipError_t launch_reduce_parts_btn(const float* partB, const float* partC, int nblk, int B, int N, int L,
                                   void* outB, void* outC, int dtype, hipStream_t st);
hipError_t launch_reduce_parts_dn(const float* part, int B, int G, int D, int N, float* out, hipStream_t st);
hipError_t launch_sens_suffix(const void* delta, int64_t sdb, int64_t sdd, StepXform stepf, const float* tile_dsum,
                              double* send, int B, int D, int L, int ntiles, int tile_len, int t_out, int dtype,
                              hipStream_t st);
hipError_t launch_tile_dsum(const void* delta, int64_t sdb, int64_t sdd, StepXform stepf, float* tile_dsum, int B,
                            int D, int L, int ntiles, int kpl, int dtype, hipStream_t st);
hipError_t launch_sens(const SensParams& p, int dtype, int kpl, hipStream_t st);
// rows of the input Jacobian: the weights (tail = false) before the main pass,
// the steps in (t0, t0 + R) (tail = true) after it
hipError_t launch_sens_rows_edge(const SensRowsParams& p, bool tail, int dtype, hipStream_t st);
hipError_t launch_sens_rows(const SensRowsParams& p, int dtype, hipStream_t st);

// ------------------------------- real, dense -------------------------------
struct DenseParams {
    const float* a; const float* b; const float* C; const float* h0;
    const float* carry_in;   // (B,D,G,N)
    const float* gy; const float* gh_last; const float* ckpt; const float* nu_in;
    float* y; float* h_last; float* ckpt_out;
    float* segP; float* segS;      // forward summaries
    float* segQ; float* segR;      // backward summaries
    float* ga; float* gb; float* gh0;
    float* partC;                  // (nblk,B,N,L)
    int B, D, L, N, nchunks, chunk, chunks_per_seg, G;
};
hipError_t launch_dense_fwd(const DenseParams& p, bool summary, hipStream_t st);
hipError_t launch_dense_bwd(const DenseParams& p, bool summary, hipStream_t st);

// ------------------------------- complex -----------------------------------
// Streams (r, phi, u, gy, y, gu, gr, gphi) are fp32 or bf16 (dtype 0 / 1; a
// complex value is an (re, im) pair of the type); parameters, states,
// checkpoints and summaries are fp32 / fp64.
struct CplxParams {
    const void* r; const void* phi; const float* lam; const float* theta;
    const void* u; const float* c; const float* h0;
    double* carry_in;        // (B,H,G,M) complex double, written by the combine pass
    const void* gy; const float* gh_last; const float* ckpt;
    double* nu_in;           // (B,H,G,M) complex double, written by the reverse combine pass
    void* y; float* h_last; float* ckpt_out;
    double* segP; double* segS; double* segQ; double* segR;   // complex double (B,H,G,M)
    void* gu; void* gr; void* gphi; float* gh0;
    double* partL; double* partT; double* partC;              // (B,G,H,M) [partC complex]
    // given transitions (SSM_COMPLEX_DENSE): a (B,H,L,M) complex64 replaces r, phi, lam,
    // theta; ga (B,H,L,M) complex64 replaces gr, gphi, glam, gtheta
    const float* a; float* ga;
    // views: r, phi (b, h) rows at b * s[0] + h * s[1]; u (b, h, t) at su[0..2] (complex
    // elements); lam, theta, c per head at h * s (0 = shared by the heads)
    int64_t sr[2], sphi[2], su[3], slam, stheta, sc;
    int B, H, L, M, nchunks, chunk, chunks_per_seg, G;
    int dtype;
};
hipError_t launch_cplx_fwd(const CplxParams& p, bool summary, hipStream_t st);
hipError_t launch_cplx_bwd(const CplxParams& p, bool summary, hipStream_t st);
hipError_t launch_cplx_combine_fwd(const CplxParams& p, hipStream_t st);
hipError_t launch_cplx_combine_rev(const CplxParams& p, hipStream_t st);
hipError_t launch_cplx_reduce(const CplxParams& p, float* glam, float* gtheta, float* gc, hipStream_t st);

struct RtrlParams {
    const void* r; const void* phi; const float* lam; const float* theta;
    const void* u; const float* c; const float* h0;
    const void* gy; const float* gh_last;
    void* y; float* glam; float* gtheta;
    double* segP;    // (B,H,G,M) complex: product of a over the segment
    double* segS;    // 3 planes (h, sl, st) of (B,H,G,M) complex: local triple from zero
    double* segRP;   // (B,H,G) x (sum r, sum phi)
    double* carry;   // 3 planes (h, sl, st) of (B,H,G,M) complex entering each segment
    double* partL; double* partT;   // (B,G,H,M)
    int64_t sr[2], sphi[2], su[3], slam, stheta, sc;   // views, as in CplxParams
    int B, H, L, M, nchunks, chunks_per_seg, G;
    int dtype;
};
hipError_t launch_cplx_rtrl(const RtrlParams& p, bool summary, hipStream_t st);
hipError_t launch_cplx_rtrl_combine(const RtrlParams& p, hipStream_t st);
hipError_t launch_cplx_rtrl_reduce(const RtrlParams& p, hipStream_t st);

// --------------------- scalar transition per head (matrix form) ------------
// Head h owns channels d = h*P + p; delta (B,H,L) rows at b*sdelta[0] +
// h*sdelta[1]; x, y (B,D,L) rows at b*s[0] + d*s[1]; A (H) at h*sA; Bm, C
// (B,L,N) at b*s[0] + t*s[2] + n.  Workspace: state (B,H,nchunks,N,P) chunk
// states (local, then entering), decay (B,H,nchunks).
struct HeadParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C; const float* h0;
    int64_t sdelta[2], sx[2], sy[2], sBm[3], sC[3], sA;
    void* y; float* h_last; float* ckpt;
    float* state; float* decay;
    int B, H, P, L, N, nchunks;
    int vx, vb, vc, vy;   // 16-byte row loads of x, B, C and 4-step stores of y are aligned
    int bstate;           // state pass of the backward: weights e^(s_u) (x = gy, Bm = C)
};
// the three passes: chunk-local states (matrix cores), the chain over chunks,
// the outputs (matrix cores; needs p.y)
hipError_t launch_head_state(const HeadParams& p, int dtype, hipStream_t st);
hipError_t launch_head_chain(const HeadParams& p, hipStream_t st);
hipError_t launch_head_out(const HeadParams& p, int dtype, hipStream_t st);
// backward of the matrix form: the chunk adjoints G_out of every chunk (reverse
// chain over the chunk sums Q_c = C^T diag(e^s) dY of the state pass), then one
// workgroup per (chunk, head, batch) for gx, gdelta and the per-head partial
// sums of gB, gC and gA
struct HeadBwdParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C; const void* gy;
    const float* ckpt;       // entering states (B, D, nchunks, N), fp32
    const float* gh_last;    // (B, D, N) or null
    int64_t sdelta[2], sx[2], sgy[2], sgx[2], sgdelta[2], sBm[3], sC[3], sA;
    float* gstate;           // (B, H, nchunks, P, N): Q_c in, G_out(c) out
    const float* decay;      // (B, H, nchunks)
    void* gx; void* gdelta; float* gh0;
    float* partB; float* partC;   // (H, B, N, L) per-head terms of gB, gC (null: not wanted)
    float* partA;                 // (H, B, nchunks) per-chunk terms of gA (null: not wanted)
    int B, H, P, L, N, nchunks;
    int vx, vgy, vb, vc;          // 16-byte row loads of x, gy, B, C are aligned
    int vgx;                      // 4-step stores of gx are aligned
};
hipError_t launch_head_rchain(const HeadBwdParams& p, hipStream_t st);
hipError_t launch_head_bwd(const HeadBwdParams& p, int dtype, hipStream_t st);
// out[h] = sum of part[h * n .. h * n + n - 1], in order
hipError_t launch_head_sum_rows(const float* part, float* out, int H, int n, hipStream_t st);

// ------------------------------- PD ----------------------------------------
struct PDParams {
    // streams (logits, d, b, C, gy, y, gd, gb, gC, ste_logits, glogits) are fp32
    // or bf16 (dtype 0 / 1); states, checkpoints and summaries are fp32
    const void* logits; const int32_t* sel_in; const int32_t* dict;
    const void* d; const void* b; const void* C; const float* h0;
    const void* gy; const float* gh_last; const float* ckpt;
    int32_t* sel_out;              // selection written by the summary pass
    const int32_t* sel;            // selection read by the later passes
    int8_t* pre;                   // (H,K,N,N) preimage lists, -1 padded
    int32_t* pre_cnt;              // (H,K,N)
    int32_t* segPi; float* segD; float* segS;   // (B,H,G,N) chunk summaries: forward local
                                                // state, or in the backward the adjoint R
    float* carry_in;               // (B,H,G,N)
    float* nu_in;                  // (B,H,G,N)
    void* y; float* h_last; float* ckpt_out;
    void* gd; void* gb; void* gC; float* gh0;
    const void* ste_logits;        // selection scores for the surrogate gradient (B,H,L,K)
    void* glogits;                 // (B,H,L,K) surrogate gradient; NULL = not wanted
    float inv_tau;                 // 1 / softmax temperature
    // views: d, b, C, logits rows (b, h) at b * s[0] + h * s[1], steps s[2] apart;
    // dictionary entry (h, k) at h * sdict[0] + k * sdict[1] (0 = shared by the heads)
    int64_t s_d[3], s_b[3], s_C[3], s_lg[3], sdict[2];
    int dense;   // d, b, C and the scores in their dense (B, H, L, N|K) layout: kernels without the stride math
    int B, H, L, N, K, chunk, G;   // G = number of chunks
    int dtype;                     // 0 fp32, 1 bf16 streams
};
hipError_t launch_pd_prep(const PDParams& p, hipStream_t st);
// out[i] = sel[i] clamped to [0, K), as the kernels read a given selection
hipError_t launch_pd_sel_copy(const int32_t* sel, int32_t* out, size_t n, int K, hipStream_t st);
hipError_t launch_pd_fwd(const PDParams& p, bool summary, hipStream_t st);
hipError_t launch_pd_combine_fwd(const PDParams& p, hipStream_t st);
hipError_t launch_pd_bwd(const PDParams& p, bool summary, hipStream_t st);
hipError_t launch_pd_combine_rev(const PDParams& p, hipStream_t st);

// ------------------------------- issue-rate probes -------------------------
// `waves` one-wave workgroups, each lane running `chains` dependency chains of
// instruction class `kind` for iters * 8 steps; sink holds waves * 64 floats.
hipError_t launch_roof(int kind, int chains, int waves, int iters, float* sink, hipStream_t st);
double roof_instrs_per_lane(int kind, int chains, int iters);

}  // namespace ssm
