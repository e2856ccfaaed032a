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
struct SelFwdParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C;
    const float* h0;        // (B,D,N) or null
    const float* carry_in;  // (B,D,G,N) state entering each segment (G > 1)
    void* y;                // (B,D,L) or null
    float* h_last;          // (B,D,N) or null
    float* ckpt;            // (B,D,ntiles,N) or null
    float* segP;            // summary pass: product of a over each segment (B,D,G,N)
    float* segS;            // summary pass: local state at segment end (B,D,G,N)
    float* tile_dsum;       // (B,D,ntiles) sum of delta over each tile, or null
    StepXform stepf;
    int B, D, L, N, ntiles, tiles_per_seg, G, vec;
};
struct SelBwdParams {
    const void* delta; const void* x; const float* A; const void* Bm; const void* C;
    const void* gy; const float* gh_last; const float* ckpt;
    const float* nu_in;     // (B,D,G,N) adjoint entering each segment from the right (G > 1)
    void* gdelta; void* gx; float* gh0;
    float* partB; float* partC;  // (nblk,B,N,L) partial sums over each block of channels
    float* partA;                // (B,G,D,N)
    float* partBias;             // (B,G,D) partial sums of the step-size bias gradient, or null
    float* segQ; float* segR;    // summary pass outputs (B,D,G,N)
    StepXform stepf;
    int B, D, L, N, ntiles, tiles_per_seg, G, vec;
};
struct SensParams {
    const void* delta; const float* A; const void* Bm; const void* C;
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
int sel_bwd_rows();  // channels per backward workgroup (one gB/gC partial per block)
hipError_t launch_seg_combine_fwd(const float* P, const float* S, const float* h0, float* carry_in,
                                  int BD, int G, int N, hipStream_t st);
hipError_t launch_seg_combine_rev(const float* Q, const float* R, const float* nu_last, float* nu_in,
                                  int BD, int G, int N, hipStream_t st);
// (nblk, B, N, L) channel-block partials of gB and/or gC (null skips) -> (B, L, N)
hipError_t launch_reduce_parts_btn(const float* partB, const float* partC, int nblk, int B, int N, int L,
                                   void* outB, void* outC, int dtype, hipStream_t st);
hipError_t launch_reduce_parts_dn(const float* part, int B, int G, int D, int N, float* out, hipStream_t st);
hipError_t launch_sens_suffix(const void* delta, StepXform stepf, const float* tile_dsum, double* send, int B, int D,
                              int L, int ntiles, int tile_len, int t_out, int dtype, hipStream_t st);
hipError_t launch_tile_dsum(const void* delta, StepXform stepf, float* tile_dsum, int B, int D, int L, int ntiles,
                            int kpl, int dtype, hipStream_t st);
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
    int B, H, L, M, nchunks, chunks_per_seg, G;
    int dtype;
};
hipError_t launch_cplx_rtrl(const RtrlParams& p, bool summary, hipStream_t st);
hipError_t launch_cplx_rtrl_combine(const RtrlParams& p, hipStream_t st);
hipError_t launch_cplx_rtrl_reduce(const RtrlParams& p, hipStream_t st);

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
