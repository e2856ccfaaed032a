// Complex diagonal scan with shared controls on gfx950 (SPARC page, abstract:
// two input-dependent scalars steer every complex mode, each mode keeping its
// own baseline rate and frequency):
//   a_{t,m} = lambda_m^{r_t} e^{i phi_t theta_m},  h_t = a_t h_{t-1} + u_t,
//   y_t = Re sum_m c_m h_{t,m}.
//
// Work mapping.  One wave per (batch, head, segment); lane m holds complex
// mode m, so the (B,H,L,M) streams u and gu move as one contiguous 512-byte
// row per step.  Complex arithmetic stays in registers.  The controls r_t,
// phi_t and gy_t of a 32-step chunk are loaded one per lane and read back per
// step with v_readlane (wave-uniform scalars).  Sums over modes (y_t and the
// per-step control gradients) are kept per step for a 32-step chunk and summed
// across the 64 lanes with one transpose-reduction per chunk.
// Segments along L run in parallel: a summary pass composes each segment's
// affine map (product of a, local state), a combine pass chains the segments,
// the main pass re-runs each segment from its exact entering state.
#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kCChunk = 32;  // checkpoint interval (steps) of the complex mode

// The recurrence runs in fp64 (the vector fp64 rate of CDNA4 equals its
// unpacked fp32 rate): for the slow modes (|a| close to 1, horizons of ~10^3
// steps) the rounding of fp32 transition factors and states accumulates to
// ~1e-6 relative, which the fp32 outputs must not inherit.  Streams,
// checkpoints and outputs stay complex64.
struct cd {
    double re, im;
};
__device__ __forceinline__ cd cmul(cd a, cd b) { return {fma(a.re, b.re, -a.im * b.im), fma(a.re, b.im, a.im * b.re)}; }
__device__ __forceinline__ cd cmul_conj_a(cd a, cd b) {  // conj(a) * b
    return {fma(a.re, b.re, a.im * b.im), fma(a.re, b.im, -a.im * b.re)};
}
__device__ __forceinline__ cd cfma(cd a, cd b, cd c) {  // a*b + c
    return {fma(a.re, b.re, fma(-a.im, b.im, c.re)), fma(a.re, b.im, fma(a.im, b.re, c.im))};
}

// a = exp(r ln(lambda)) (cos w + i sin w), w = phi * theta (exact in double:
// the product of two floats fits in the 53-bit mantissa).
__device__ __forceinline__ cd trans_a(float r, double lnlam, float phi, float th) {
    const double mag = exp((double)r * lnlam);
    double s, c;
    sincos((double)phi * (double)th, &s, &c);
    return {mag * c, mag * s};
}

__device__ __forceinline__ float lanev(float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); }

struct CUnit {
    int s, g, b, hh, m, mc;
    bool act;
};
__device__ __forceinline__ bool cunit(const CplxParams& p, CUnit& u) {
    const int wave = threadIdx.x >> 6;
    const int unit = blockIdx.x * 4 + wave;
    if (unit >= p.B * p.H * p.G) return false;
    u.s = unit / p.G;
    u.g = unit - u.s * p.G;
    u.b = u.s / p.H;
    u.hh = u.s - u.b * p.H;
    u.m = threadIdx.x & 63;
    u.act = u.m < p.M;
    u.mc = u.act ? u.m : p.M - 1;
    return true;
}

// ---------------------------------------------------------------------------
// forward.  SUMMARY: per segment the map h_end = P h_start + S (h_start = 0).
// ---------------------------------------------------------------------------
template <bool SUMMARY>
__global__ __launch_bounds__(256) void cplx_fwd_kernel(CplxParams p) {
    CUnit u;
    if (!cunit(p, u)) return;
    const int L = p.L, M = p.M;
    const size_t pm = (size_t)u.hh * M + u.mc;
    const double lnl = log((double)p.lam[pm]);
    const float th = p.theta[pm];
    const double c_re = p.c[2 * pm], c_im = p.c[2 * pm + 1];
    const size_t us = ((size_t)u.s * p.G + u.g) * M + u.mc;  // (B*H, G, M)
    cd h = {0.0, 0.0}, P = {1.0, 0.0};
    if (!SUMMARY) {
        if (p.G > 1) h = {p.carry_in[2 * us], p.carry_in[2 * us + 1]};
        else if (p.h0) h = {p.h0[2 * ((size_t)u.s * M + u.mc)], p.h0[2 * ((size_t)u.s * M + u.mc) + 1]};
        if (!u.act) h = {0.0, 0.0};
    }
    const int c0 = u.g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const float* urow = p.u + (size_t)u.s * L * M * 2;
    for (int ch = c0; ch < c1; ++ch) {
        const int t0 = ch * kCChunk;
        if (!SUMMARY && p.ckpt_out && u.act) {
            const size_t o = ((size_t)u.s * p.nchunks + ch) * M + u.m;
            p.ckpt_out[2 * o] = (float)h.re;
            p.ckpt_out[2 * o + 1] = (float)h.im;
        }
        const int tl = t0 + (u.m & 31);
        const bool tv = tl < L;
        const float rv = tv ? p.r[(size_t)u.s * L + tl] : 0.0f;
        const float pv = tv ? p.phi[(size_t)u.s * L + tl] : 0.0f;
        float yp[kCChunk];
#pragma unroll
        for (int j = 0; j < kCChunk; ++j) {
            const int t = t0 + j;
            yp[j] = 0.0f;
            if (t < L) {  // uniform
                const cd a = trans_a(lanev(rv, j), lnl, lanev(pv, j), th);
                cd ut = {0.0, 0.0};
                if (u.act) ut = {urow[((size_t)t * M + u.m) * 2], urow[((size_t)t * M + u.m) * 2 + 1]};
                h = cfma(a, h, ut);
                if (SUMMARY) P = cmul(a, P);
                else yp[j] = (float)fma(c_re, h.re, -c_im * h.im);
            }
        }
        if (!SUMMARY && p.y) {
            const float ys = wave_transpose_sum32(yp);
            const int t = t0 + (u.m >> 1);
            if ((u.m & 1) == 0 && t < L) p.y[(size_t)u.s * L + t] = ys;
        }
    }
    if (!u.act) return;
    if (SUMMARY) {
        p.segP[2 * us] = P.re;
        p.segP[2 * us + 1] = P.im;
        p.segS[2 * us] = h.re;
        p.segS[2 * us + 1] = h.im;
    } else if (p.h_last && u.g == p.G - 1) {
        const size_t o = (size_t)u.s * M + u.m;
        p.h_last[2 * o] = (float)h.re;
        p.h_last[2 * o + 1] = (float)h.im;
    }
}

// ---------------------------------------------------------------------------
// backward.  nu_t = conj(a_t) mu_t with mu_t = gy_t conj(c) + nu_{t+1}
// (nu_L = gh_last), g_u = mu, g_a = mu conj(h_{t-1}), g_z = conj(a) g_a;
//   gr_t = sum_m Re g_z ln(lambda),   gphi_t = sum_m Im g_z theta,
//   g ln(lambda) += Re g_z r_t,  gtheta += Im g_z phi_t,  gc += gy conj(h_t).
// Reverse over the chunks of a segment; each chunk's states are recomputed
// (in fp64, from its checkpoint) and kept in registers as complex64.
// SUMMARY: per segment the adjoint map nu_start = Q nu_end + R.
// ---------------------------------------------------------------------------
template <bool SUMMARY>
__global__ __launch_bounds__(256) void cplx_bwd_kernel(CplxParams p) {
    CUnit u;
    if (!cunit(p, u)) return;
    const int L = p.L, M = p.M;
    const size_t pm = (size_t)u.hh * M + u.mc;
    const double lnl = log((double)p.lam[pm]);
    const float th = p.theta[pm];
    const double cjr = p.c[2 * pm], cji = -(double)p.c[2 * pm + 1];  // conj(c)
    const size_t us = ((size_t)u.s * p.G + u.g) * M + u.mc;
    cd nu = {0.0, 0.0}, Q = {1.0, 0.0};
    if (!SUMMARY) {
        if (p.G > 1) nu = {p.nu_in[2 * us], p.nu_in[2 * us + 1]};
        else if (p.gh_last) nu = {p.gh_last[2 * ((size_t)u.s * M + u.mc)], p.gh_last[2 * ((size_t)u.s * M + u.mc) + 1]};
        if (!u.act) nu = {0.0, 0.0};
    }
    double gl = 0.0, gt = 0.0, gcr = 0.0, gci = 0.0;
    const int c0 = u.g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const float* urow = p.u + (size_t)u.s * L * M * 2;
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const int t0 = ch * kCChunk;
        const int tl = t0 + (u.m & 31);
        const bool tv = tl < L;
        const float rv = tv ? p.r[(size_t)u.s * L + tl] : 0.0f;
        const float pv = tv ? p.phi[(size_t)u.s * L + tl] : 0.0f;
        const float gv = tv ? p.gy[(size_t)u.s * L + tl] : 0.0f;
        if (SUMMARY) {
#pragma unroll
            for (int j = kCChunk - 1; j >= 0; --j) {
                if (t0 + j < L) {
                    const cd a = trans_a(lanev(rv, j), lnl, lanev(pv, j), th);
                    const double g = lanev(gv, j);
                    const cd mu = {fma(g, cjr, nu.re), fma(g, cji, nu.im)};
                    nu = cmul_conj_a(a, mu);
                    Q = cmul_conj_a(a, Q);
                }
            }
            continue;
        }
        // recompute the chunk's states from its checkpoint
        float hre[kCChunk + 1], him[kCChunk + 1];
        cd hcur;
        {
            const size_t o = ((size_t)u.s * p.nchunks + ch) * M + u.mc;
            hcur = {p.ckpt[2 * o], p.ckpt[2 * o + 1]};
            hre[0] = (float)hcur.re;
            him[0] = (float)hcur.im;
        }
#pragma unroll
        for (int j = 0; j < kCChunk; ++j) {
            if (t0 + j < L) {
                const cd a = trans_a(lanev(rv, j), lnl, lanev(pv, j), th);
                cd ut = {0.0, 0.0};
                if (u.act) ut = {urow[((size_t)(t0 + j) * M + u.m) * 2], urow[((size_t)(t0 + j) * M + u.m) * 2 + 1]};
                hcur = cfma(a, hcur, ut);
            }
            hre[j + 1] = (float)hcur.re;
            him[j + 1] = (float)hcur.im;
        }
        // reverse in two halves of 16 steps; the per-step sums over modes of
        // terms that cancel strongly are formed in fp64
#pragma unroll
        for (int half = kCChunk / 16 - 1; half >= 0; --half) {
            double grp[16], gpp[16];
#pragma unroll
            for (int jj = 15; jj >= 0; --jj) {
                const int j = 16 * half + jj;
                grp[jj] = 0.0;
                gpp[jj] = 0.0;
                const int t = t0 + j;
                if (t < L) {
                    const float rj = lanev(rv, j), pj = lanev(pv, j);
                    const double g = lanev(gv, j);
                    const cd a = trans_a(rj, lnl, pj, th);
                    const cd mu = {fma(g, cjr, nu.re), fma(g, cji, nu.im)};
                    if (p.gu && u.act) {
                        float* dst = p.gu + (((size_t)u.s * L + t) * M + u.m) * 2;
                        dst[0] = (float)mu.re;
                        dst[1] = (float)mu.im;
                    }
                    const cd ga = cmul(mu, cd{hre[j], -(double)him[j]});
                    const cd gz = cmul_conj_a(a, ga);
                    if (u.act) {
                        grp[jj] = gz.re * lnl;
                        gpp[jj] = gz.im * th;
                        gl = fma(gz.re, (double)rj, gl);
                        gt = fma(gz.im, (double)pj, gt);
                        gcr = fma(g, (double)hre[j + 1], gcr);
                        gci = fma(-g, (double)him[j + 1], gci);
                    }
                    nu = cmul_conj_a(a, mu);
                }
            }
            const double sr = wave_transpose_sum16_f64(grp);
            const double sp = wave_transpose_sum16_f64(gpp);
            const int t = t0 + 16 * half + (u.m >> 2);
            if ((u.m & 3) == 0 && t < L) {
                if (p.gr) p.gr[(size_t)u.s * L + t] = (float)sr;
                if (p.gphi) p.gphi[(size_t)u.s * L + t] = (float)sp;
            }
        }
    }
    if (!u.act) return;
    if (SUMMARY) {
        p.segQ[2 * us] = Q.re;
        p.segQ[2 * us + 1] = Q.im;
        p.segR[2 * us] = nu.re;
        p.segR[2 * us + 1] = nu.im;
        return;
    }
    if (p.gh0 && u.g == 0) {
        const size_t o = (size_t)u.s * M + u.m;
        p.gh0[2 * o] = (float)nu.re;
        p.gh0[2 * o + 1] = (float)nu.im;
    }
    // per-(batch, segment) partial sums of the mode-parameter gradients, (B,G,H,M)
    const size_t po = (((size_t)u.b * p.G + u.g) * p.H + u.hh) * M + u.m;
    if (p.partL) p.partL[po] = gl;
    if (p.partT) p.partT[po] = gt;
    if (p.partC) {
        p.partC[2 * po] = gcr;
        p.partC[2 * po + 1] = gci;
    }
}

// segment combines, one thread per (sequence, mode)
__global__ void cplx_combine_fwd_kernel(CplxParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.H * p.M) return;
    const int s = i / p.M, m = i - s * p.M;
    cd h = {0.0, 0.0};
    if (p.h0) h = {p.h0[2 * (size_t)i], p.h0[2 * (size_t)i + 1]};
    for (int g = 0; g < p.G; ++g) {
        const size_t o = ((size_t)s * p.G + g) * p.M + m;
        p.carry_in[2 * o] = h.re;
        p.carry_in[2 * o + 1] = h.im;
        h = cfma({p.segP[2 * o], p.segP[2 * o + 1]}, h, {p.segS[2 * o], p.segS[2 * o + 1]});
    }
}
__global__ void cplx_combine_rev_kernel(CplxParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.H * p.M) return;
    const int s = i / p.M, m = i - s * p.M;
    cd v = {0.0, 0.0};
    if (p.gh_last) v = {p.gh_last[2 * (size_t)i], p.gh_last[2 * (size_t)i + 1]};
    for (int g = p.G - 1; g >= 0; --g) {
        const size_t o = ((size_t)s * p.G + g) * p.M + m;
        p.nu_in[2 * o] = v.re;
        p.nu_in[2 * o + 1] = v.im;
        v = cfma({p.segQ[2 * o], p.segQ[2 * o + 1]}, v, {p.segR[2 * o], p.segR[2 * o + 1]});
    }
}
// (B,G,H,M) partials -> (H,M): one wave per (head, mode); lane l adds the
// partials l, l+64, ... in order, then a fixed butterfly over the 64 lanes.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_d<SSM_DPP_QUAD(1, 0, 3, 2)>(v);
    v += dpp_d<SSM_DPP_QUAD(2, 3, 0, 1)>(v);
    v += dpp_d<SSM_DPP_ROW_HALF_MIRROR>(v);
    v += dpp_d<SSM_DPP_ROW_MIRROR>(v);
    double w = v;
    permswap_d<false>(v, w);  // rows 0<->1, 2<->3
    v += w;
    w = v;
    permswap_d<true>(v, w);   // halves
    return v + w;
}
__global__ __launch_bounds__(256) void cplx_reduce_kernel(CplxParams p, float* glam, float* gtheta, float* gc) {
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int HM = p.H * p.M;
    if (i >= HM) return;  // whole waves leave together
    const int lane = threadIdx.x & 63;
    double sl = 0.0, st = 0.0, cr = 0.0, ci = 0.0;
    for (int k = lane; k < p.B * p.G; k += 64) {
        const size_t o = (size_t)k * HM + i;
        sl += p.partL[o];
        st += p.partT[o];
        cr += p.partC[2 * o];
        ci += p.partC[2 * o + 1];
    }
    sl = wave_sum_f64(sl);
    st = wave_sum_f64(st);
    cr = wave_sum_f64(cr);
    ci = wave_sum_f64(ci);
    if (lane != 0) return;
    if (glam) glam[i] = (float)(sl / (double)p.lam[i]);  // d/d lambda = (d/d ln lambda) / lambda
    if (gtheta) gtheta[i] = (float)st;
    if (gc) {
        gc[2 * i] = (float)cr;
        gc[2 * i + 1] = (float)ci;
    }
}

hipError_t launch_cplx_fwd(const CplxParams& p, bool summary, hipStream_t st) {
    const int units = p.B * p.H * p.G;
    dim3 grid((units + 3) / 4), block(256);
    if (summary) cplx_fwd_kernel<true><<<grid, block, 0, st>>>(p);
    else cplx_fwd_kernel<false><<<grid, block, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_cplx_bwd(const CplxParams& p, bool summary, hipStream_t st) {
    const int units = p.B * p.H * p.G;
    dim3 grid((units + 3) / 4), block(256);
    if (summary) cplx_bwd_kernel<true><<<grid, block, 0, st>>>(p);
    else cplx_bwd_kernel<false><<<grid, block, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_cplx_combine_fwd(const CplxParams& p, hipStream_t st) {
    const int n = p.B * p.H * p.M;
    cplx_combine_fwd_kernel<<<(n + 255) / 256, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_cplx_combine_rev(const CplxParams& p, hipStream_t st) {
    const int n = p.B * p.H * p.M;
    cplx_combine_rev_kernel<<<(n + 255) / 256, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_cplx_reduce(const CplxParams& p, float* glam, float* gtheta, float* gc, hipStream_t st) {
    const int n = p.H * p.M;
    cplx_reduce_kernel<<<(n + 3) / 4, 256, 0, st>>>(p, glam, gtheta, gc);
    return hipGetLastError();
}

}  // namespace ssm
