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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ssm {

constexpr int kCChunk = 32;  // checkpoint interval (steps) of the complex mode

// The recurrence runs in fp64 (the vector fp64 rate of CDNA4 is half its
// fp32 rate): for the slow modes (|a| close to 1, horizons of ~10^3
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

// Double-precision exp and sincos for the transition factors, written out
// from their series (the library routines also carry large-argument paths
// that cost more than the whole recurrence step).  Constants: ln 2 and pi/2
// split into a head with trailing zero bits (so k * head is exact) and a
// tail, each part the correctly rounded value of the exact remainder.
constexpr double kLog2eD = 0x1.71547652b82fep+0;   // 1 / ln 2
constexpr double kLn2Hi = 0x1.62e42ff000000p-1;    // ln 2, first 29 bits
constexpr double kLn2Lo = -0x1.718432a1b0e26p-35;  // ln 2 - kLn2Hi
constexpr double k2OverPi = 0x1.45f306dc9c883p-1;  // 2 / pi
constexpr double kPio2A = 0x1.921fb54400000p+0;    // pi/2, first 33 bits
constexpr double kPio2B = 0x1.0b4611a600000p-34;   // next 33 bits
constexpr double kPio2C = 0x1.3198a2e037073p-69;   // remainder

// exp(x) = 2^k exp(f), x = k ln 2 + f, |f| <= ln2 / 2; exp(f) by its Taylor
// series through f^11 (truncation below 7e-15 relative: a factor's error then
// stays below 1e-10 relative after 10^4 steps, far inside the fp32 outputs'
// tolerance, while the state itself still accumulates in double).
__device__ __forceinline__ double exp_d(double x) {
    const double k = fmin(fmax(rint(x * kLog2eD), -1100.0), 1100.0);
    double f = fma(-k, kLn2Hi, x);
    f = fma(-k, kLn2Lo, f);
    double e = 1.0 / 39916800.0;          // 1/11!
    e = fma(e, f, 1.0 / 3628800.0);       // 1/10!
    e = fma(e, f, 1.0 / 362880.0);        // 1/9!
    e = fma(e, f, 1.0 / 40320.0);         // 1/8!
    e = fma(e, f, 1.0 / 5040.0);          // 1/7!
    e = fma(e, f, 1.0 / 720.0);           // 1/6!
    e = fma(e, f, 1.0 / 120.0);           // 1/5!
    e = fma(e, f, 1.0 / 24.0);            // 1/4!
    e = fma(e, f, 1.0 / 6.0);             // 1/3!
    e = fma(e, f, 0.5);
    e = fma(e, f, 1.0);
    e = fma(e, f, 1.0);
    return ldexp(e, (int)k);
}

// sin w and cos w for |w| <= kFastTrig: w = q pi/2 + r with |r| <= pi/4
// (three-part reduction, exact products for |q| < 2^20), Taylor series of
// sin r through r^13 and of cos r through r^14 (truncation below 3e-14 and
// 1e-15), then the quadrant q mod 4.  Larger arguments use the library routine
// (chosen per chunk, see trans_a).
constexpr double kFastTrig = 1.0e6;
__device__ __forceinline__ void sincos_d(double w, double* sp, double* cp) {
    const double q = rint(w * k2OverPi);
    double r = fma(-q, kPio2A, w);
    r = fma(-q, kPio2B, r);
    r = fma(-q, kPio2C, r);
    const double r2 = r * r;
    double ps = 1.0 / 6227020800.0;               // 1/13!
    ps = fma(ps, r2, -1.0 / 39916800.0);          // -1/11!
    ps = fma(ps, r2, 1.0 / 362880.0);             // 1/9!
    ps = fma(ps, r2, -1.0 / 5040.0);              // -1/7!
    ps = fma(ps, r2, 1.0 / 120.0);                // 1/5!
    ps = fma(ps, r2, -1.0 / 6.0);                 // -1/3!
    const double sr = fma(r * r2, ps, r);
    double pc = -1.0 / 87178291200.0;             // -1/14!
    pc = fma(pc, r2, 1.0 / 479001600.0);          // 1/12!
    pc = fma(pc, r2, -1.0 / 3628800.0);           // -1/10!
    pc = fma(pc, r2, 1.0 / 40320.0);              // 1/8!
    pc = fma(pc, r2, -1.0 / 720.0);               // -1/6!
    pc = fma(pc, r2, 1.0 / 24.0);                 // 1/4!
    pc = fma(pc, r2, -0.5);                       // -1/2!
    const double cr = fma(r2, pc, 1.0);
    const int n = (int)q & 3;
    const double s1 = (n & 1) ? cr : sr, c1 = (n & 1) ? sr : cr;
    *sp = (n & 2) ? -s1 : s1;
    *cp = ((n + 1) & 2) ? -c1 : c1;
}

// a = exp(r ln(lambda)) (cos w + i sin w), w = phi * theta (exact in double:
// the product of two floats fits in the 53-bit mantissa).  FAST: every
// |w| of the chunk is at most kFastTrig.
template <bool FAST>
__device__ __forceinline__ cd trans_a(float r, double lnlam, float phi, float th) {
    const double mag = exp_d((double)r * lnlam);
    double s, c;
    if (FAST) sincos_d((double)phi * (double)th, &s, &c);
    else sincos((double)phi * (double)th, &s, &c);
    return {mag * c, mag * s};
}

// Wave maximum of |x| (all 64 lanes).
__device__ __forceinline__ float wave_absmax(float x) {
    float m = fabsf(x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    return m;
}
// Run body(FAST, FULL) for one chunk: FAST when no phase argument of the
// chunk can exceed kFastTrig, FULL when all kCChunk steps lie inside L.
template <typename F>
__device__ __forceinline__ void cplx_chunk(float pv, float thmax, bool full, F&& body) {
    const bool fast = !__any((double)fabsf(pv) * (double)thmax > kFastTrig);
    if (fast) {
        if (full) body(std::true_type{}, std::true_type{});
        else body(std::true_type{}, std::false_type{});
    } else {
        body(std::false_type{}, std::false_type{});
    }
}

__device__ __forceinline__ float lanev(float v, int j) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j)); }

// u of steps t0 .. t0+K-1 for mode mc (complex64); zero past L and on idle
// lanes.  A block inside the sequence loads unconditionally, so all K loads
// are in flight before the first step runs.
// One complex value of a stream: an (re, im) pair of fp32 or of bf16.
template <typename T> struct CPair;
template <> struct CPair<float> {
    using V = float2;
    __device__ static float2 widen(float2 v) { return v; }
    __device__ static float2 narrow(float re, float im) { return make_float2(re, im); }
};
template <> struct CPair<bf16_t> {
    using V = uint32_t;   // re in the low half, im in the high half
    __device__ static float2 widen(uint32_t v) {
        return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
    }
    __device__ static uint32_t narrow(float re, float im) {
        return (uint32_t)from_f32<bf16_t>(re) | ((uint32_t)from_f32<bf16_t>(im) << 16);
    }
};

// K steps of mode mc from t0 of a (step, mode) slice whose steps are sl
// complex elements apart (modes contiguous)
template <typename T, int K>
__device__ __forceinline__ void load_u(const T* __restrict__ urow, int t0, int L, int64_t sl, int mc, bool act,
                                       float2 (&v)[K]) {
    using V = typename CPair<T>::V;
    const V* __restrict__ q = reinterpret_cast<const V*>(urow) + (int64_t)t0 * sl + mc;
    if (t0 + K <= L) {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = CPair<T>::widen(q[(int64_t)j * sl]);
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j)
            v[j] = t0 + j < L ? CPair<T>::widen(q[(int64_t)j * sl]) : make_float2(0.0f, 0.0f);
    }
    if (!act) {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = make_float2(0.0f, 0.0f);
    }
}

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
// DENSE: the transitions a_t are given (SSM_COMPLEX_DENSE, complex64 streams)
// and loaded like u instead of being formed from the controls.
template <typename T, bool SUMMARY, bool DENSE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void cplx_fwd_kernel(CplxParams p) {
    CUnit u;
    if (!cunit(p, u)) return;
    const int L = p.L, M = p.M;
    const double lnl = DENSE ? 0.0 : log((double)p.lam[(int64_t)u.hh * p.slam + u.mc]);
    const float th = DENSE ? 0.0f : p.theta[(int64_t)u.hh * p.stheta + u.mc];
    const int64_t pc = (int64_t)u.hh * p.sc + u.mc;
    const double c_re = p.c[2 * pc], c_im = p.c[2 * pc + 1];
    const float thmax = DENSE ? 0.0f : wave_absmax(th);
    const size_t us = ((size_t)u.s * p.G + u.g) * M + u.mc;  // (B*H, G, M)
    cd h = {0.0, 0.0}, P = {1.0, 0.0};
    if (!SUMMARY) {
        if (p.G > 1) h = {p.carry_in[2 * us], p.carry_in[2 * us + 1]};
        else if (p.h0) h = {p.h0[2 * ((size_t)u.s * M + u.mc)], p.h0[2 * ((size_t)u.s * M + u.mc) + 1]};
        if (!u.act) h = {0.0, 0.0};
    }
    const int c0 = u.g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const T* urow = (const T*)p.u + 2 * ((int64_t)u.b * p.su[0] + (int64_t)u.hh * p.su[1]);
    const T* arow = DENSE ? (const T*)p.a + (size_t)u.s * L * M * 2 : nullptr;
    const T* rrow = (const T*)p.r + ((int64_t)u.b * p.sr[0] + (int64_t)u.hh * p.sr[1]);
    const T* prow = (const T*)p.phi + ((int64_t)u.b * p.sphi[0] + (int64_t)u.hh * p.sphi[1]);
    for (int ch = c0; ch < c1; ++ch) {
        const int t0 = ch * kCChunk;
        if (!SUMMARY && p.ckpt_out && u.act) {
            const size_t o = ((size_t)u.s * p.nchunks + ch) * M + u.m;
            p.ckpt_out[2 * o] = (float)h.re;
            p.ckpt_out[2 * o + 1] = (float)h.im;
        }
        const int tl = t0 + (u.m & 31);
        const bool tv = tl < L;
        const float rv = (tv && !DENSE) ? to_f32(rrow[tl]) : 0.0f;
        const float pv = (tv && !DENSE) ? to_f32(prow[tl]) : 0.0f;
        float yp[kCChunk];
        auto body = [&](auto fastc, auto fullc) {
            constexpr bool FAST = decltype(fastc)::value, FULL = decltype(fullc)::value;
#pragma unroll
            for (int hb = 0; hb < kCChunk / 16; ++hb) {
                float2 uv[16], av[16];
                load_u<T, 16>(urow, t0 + 16 * hb, L, p.su[2], u.mc, u.act, uv);
                if (DENSE) load_u<T, 16>(arow, t0 + 16 * hb, L, M, u.mc, u.act, av);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int j = 16 * hb + jj;
                    yp[j] = 0.0f;
                    if (FULL || t0 + j < L) {  // uniform
                        const cd a = DENSE ? cd{av[jj].x, av[jj].y} : trans_a<FAST>(lanev(rv, j), lnl, lanev(pv, j), th);
                        h = cfma(a, h, cd{uv[jj].x, uv[jj].y});
                        if (SUMMARY) P = cmul(a, P);
                        else yp[j] = (float)fma(c_re, h.re, -c_im * h.im);
                    }
                }
            }
        };
        if constexpr (DENSE) {
            if (t0 + kCChunk <= L) body(std::true_type{}, std::true_type{});
            else body(std::true_type{}, std::false_type{});
        } else {
            cplx_chunk(pv, thmax, t0 + kCChunk <= L, body);
        }
        if (!SUMMARY && p.y) {
            const float ys = wave_transpose_sum32(yp);
            const int t = t0 + (u.m >> 1);
            if ((u.m & 1) == 0 && t < L) ((T*)p.y)[(size_t)u.s * L + t] = from_f32<T>(ys);
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
// DENSE: given transitions; g_a is written per step and mode instead of the
// control and mode-parameter gradients.
// ---------------------------------------------------------------------------
template <typename T, bool SUMMARY, bool DENSE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void cplx_bwd_kernel(CplxParams p) {
    CUnit u;
    if (!cunit(p, u)) return;
    const int L = p.L, M = p.M;
    const double lnl = DENSE ? 0.0 : log((double)p.lam[(int64_t)u.hh * p.slam + u.mc]);
    const float th = DENSE ? 0.0f : p.theta[(int64_t)u.hh * p.stheta + u.mc];
    const int64_t pc = (int64_t)u.hh * p.sc + u.mc;
    const double cjr = p.c[2 * pc], cji = -(double)p.c[2 * pc + 1];  // conj(c)
    const float thmax = DENSE ? 0.0f : wave_absmax(th);
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
    const T* urow = (const T*)p.u + 2 * ((int64_t)u.b * p.su[0] + (int64_t)u.hh * p.su[1]);
    const T* arow = DENSE ? (const T*)p.a + (size_t)u.s * L * M * 2 : nullptr;
    const T* rrow = (const T*)p.r + ((int64_t)u.b * p.sr[0] + (int64_t)u.hh * p.sr[1]);
    const T* prow = (const T*)p.phi + ((int64_t)u.b * p.sphi[0] + (int64_t)u.hh * p.sphi[1]);
    for (int ch = c1 - 1; ch >= c0; --ch) {
        const int t0 = ch * kCChunk;
        const int tl = t0 + (u.m & 31);
        const bool tv = tl < L;
        const float rv = (tv && !DENSE) ? to_f32(rrow[tl]) : 0.0f;
        const float pv = (tv && !DENSE) ? to_f32(prow[tl]) : 0.0f;
        const float gv = tv ? to_f32(((const T*)p.gy)[(size_t)u.s * L + tl]) : 0.0f;
        auto body = [&](auto fastc, auto fullc) {
        constexpr bool FAST = decltype(fastc)::value, FULL = decltype(fullc)::value;
        if (SUMMARY) {
#pragma unroll
            for (int half = kCChunk / 16 - 1; half >= 0; --half) {
                float2 av[16];
                if (DENSE) load_u<T, 16>(arow, t0 + 16 * half, L, M, u.mc, u.act, av);
#pragma unroll
                for (int jj = 15; jj >= 0; --jj) {
                    const int j = 16 * half + jj;
                    if (FULL || t0 + j < L) {
                        const cd a = DENSE ? cd{av[jj].x, av[jj].y} : trans_a<FAST>(lanev(rv, j), lnl, lanev(pv, j), th);
                        const double g = lanev(gv, j);
                        const cd mu = {fma(g, cjr, nu.re), fma(g, cji, nu.im)};
                        nu = cmul_conj_a(a, mu);
                        Q = cmul_conj_a(a, Q);
                    }
                }
            }
            return;
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
        for (int hb = 0; hb < kCChunk / 16; ++hb) {
            float2 uv[16], av[16];
            load_u<T, 16>(urow, t0 + 16 * hb, L, p.su[2], u.mc, u.act, uv);
            if (DENSE) load_u<T, 16>(arow, t0 + 16 * hb, L, M, u.mc, u.act, av);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = 16 * hb + jj;
                if (FULL || t0 + j < L) {
                    const cd a = DENSE ? cd{av[jj].x, av[jj].y} : trans_a<FAST>(lanev(rv, j), lnl, lanev(pv, j), th);
                    hcur = cfma(a, hcur, cd{uv[jj].x, uv[jj].y});
                }
                hre[j + 1] = (float)hcur.re;
                him[j + 1] = (float)hcur.im;
            }
        }
        // reverse in two halves of 16 steps; the per-step sums over modes of
        // terms that cancel strongly are formed in fp64
#pragma unroll
        for (int half = kCChunk / 16 - 1; half >= 0; --half) {
            double grp[16], gpp[16];
            float2 av[16];  // the half's transitions again (just read: cache hits)
            if (DENSE) load_u<T, 16>(arow, t0 + 16 * half, L, M, u.mc, u.act, av);
#pragma unroll
            for (int jj = 15; jj >= 0; --jj) {
                const int j = 16 * half + jj;
                grp[jj] = 0.0;
                gpp[jj] = 0.0;
                const int t = t0 + j;
                if (FULL || t < L) {
                    const float rj = lanev(rv, j), pj = lanev(pv, j);
                    const double g = lanev(gv, j);
                    const cd a = DENSE ? cd{av[jj].x, av[jj].y} : trans_a<FAST>(rj, lnl, pj, th);
                    const cd mu = {fma(g, cjr, nu.re), fma(g, cji, nu.im)};
                    if (p.gu && u.act)
                        reinterpret_cast<typename CPair<T>::V*>(p.gu)[((size_t)u.s * L + t) * M + u.m] =
                            CPair<T>::narrow((float)mu.re, (float)mu.im);
                    if (DENSE) {
                        const cd ga = cmul(mu, cd{hre[j], -(double)him[j]});
                        if (p.ga && u.act)
                            reinterpret_cast<float2*>(p.ga)[((size_t)u.s * L + t) * M + u.m] =
                                make_float2((float)ga.re, (float)ga.im);
                        if (u.act) {
                            gcr = fma(g, (double)hre[j + 1], gcr);
                            gci = fma(-g, (double)him[j + 1], gci);
                        }
                        nu = cmul_conj_a(a, mu);
                        continue;
                    }
                    // g_z = conj(a) mu conj(h_{t-1}) = nu_t conj(h_{t-1}): one product on the new adjoint
                    const cd nun = cmul_conj_a(a, mu);
                    const cd gz = cmul(nun, cd{hre[j], -(double)him[j]});
                    if (u.act) {
                        grp[jj] = gz.re * lnl;
                        gpp[jj] = gz.im * th;
                        gl = fma(gz.re, (double)rj, gl);
                        gt = fma(gz.im, (double)pj, gt);
                        gcr = fma(g, (double)hre[j + 1], gcr);
                        gci = fma(-g, (double)him[j + 1], gci);
                    }
                    nu = nun;
                }
            }
            if (DENSE) continue;
            const double sr = wave_transpose_sum16_f64(grp);
            const double sp = wave_transpose_sum16_f64(gpp);
            const int t = t0 + 16 * half + (u.m >> 2);
            if ((u.m & 3) == 0 && t < L) {
                if (p.gr) ((T*)p.gr)[(size_t)u.s * L + t] = from_f32<T>((float)sr);
                if (p.gphi) ((T*)p.gphi)[(size_t)u.s * L + t] = from_f32<T>((float)sp);
            }
        }
        };
        if constexpr (DENSE) {
            if (t0 + kCChunk <= L) body(std::true_type{}, std::true_type{});
            else body(std::true_type{}, std::false_type{});
        } else {
            cplx_chunk(pv, thmax, t0 + kCChunk <= L, body);
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

// complex value i of an interleaved (re, im) fp64 array, as one 16-byte access
__device__ __forceinline__ cd ld_cd(const double* base, size_t i) {
    const double2 v = reinterpret_cast<const double2*>(base)[i];
    return {v.x, v.y};
}
__device__ __forceinline__ void st_cd(double* base, size_t i, cd v) {
    reinterpret_cast<double2*>(base)[i] = make_double2(v.re, v.im);
}

// segment combines, one thread per (sequence, mode)
constexpr int kCombBatch = 8;
__global__ __launch_bounds__(256) void cplx_combine_fwd_kernel(CplxParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.H * p.M) return;
    const int s = i / p.M, m = i - s * p.M;
    cd h = {0.0, 0.0};
    if (p.h0) h = {p.h0[2 * (size_t)i], p.h0[2 * (size_t)i + 1]};
    // summaries are loaded kCombBatch segments at a time, all in flight before
    // the chain consumes them
    const size_t o0 = (size_t)s * p.G * p.M + m;
    for (int g0 = 0; g0 < p.G; g0 += kCombBatch) {
        cd P[kCombBatch], S[kCombBatch];
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g0 + j < p.G) {
                P[j] = ld_cd(p.segP, o0 + (size_t)(g0 + j) * p.M);
                S[j] = ld_cd(p.segS, o0 + (size_t)(g0 + j) * p.M);
            }
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g0 + j < p.G) {
                st_cd(p.carry_in, o0 + (size_t)(g0 + j) * p.M, h);
                h = cfma(P[j], h, S[j]);
            }
    }
}
__global__ __launch_bounds__(256) void cplx_combine_rev_kernel(CplxParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.H * p.M) return;
    const int s = i / p.M, m = i - s * p.M;
    cd v = {0.0, 0.0};
    if (p.gh_last) v = {p.gh_last[2 * (size_t)i], p.gh_last[2 * (size_t)i + 1]};
    const size_t o0 = (size_t)s * p.G * p.M + m;
    for (int g1 = p.G - 1; g1 >= 0; g1 -= kCombBatch) {
        cd Q[kCombBatch], R[kCombBatch];
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g1 - j >= 0) {
                Q[j] = ld_cd(p.segQ, o0 + (size_t)(g1 - j) * p.M);
                R[j] = ld_cd(p.segR, o0 + (size_t)(g1 - j) * p.M);
            }
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g1 - j >= 0) {
                st_cd(p.nu_in, o0 + (size_t)(g1 - j) * p.M, v);
                v = cfma(Q[j], v, R[j]);
            }
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
        if (p.partL) sl += p.partL[o];  // uniform: absent for given transitions
        if (p.partT) st += p.partT[o];
        if (p.partC) {
            cr += p.partC[2 * o];
            ci += p.partC[2 * o + 1];
        }
    }
    sl = wave_sum_f64(sl);
    st = wave_sum_f64(st);
    cr = wave_sum_f64(cr);
    ci = wave_sum_f64(ci);
    if (lane != 0) return;
    if (glam) glam[i] = (float)(sl / (double)p.lam[(int64_t)(i / p.M) * p.slam + i % p.M]);  // d/d ln lambda / lambda
    if (gtheta) gtheta[i] = (float)st;
    if (gc) {
        gc[2 * i] = (float)cr;
        gc[2 * i + 1] = (float)ci;
    }
}

// ---------------------------------------------------------------------------
// Forward-mode (real-time recurrent) gradients w.r.t. lambda and theta (SPARC
// page, abstract: exact recurrent learning for the structured recurrence).
// With a_t = exp(r_t ln lambda + i phi_t theta): da/dlambda = a r_t / lambda and
// da/dtheta = i phi_t a, so the state sensitivities obey the same diagonal
// recurrence as h:
//   sl_t = a_t sl_{t-1} + (r_t / lambda) a_t h_{t-1},  st_t = a_t st_{t-1} + i phi_t a_t h_{t-1},
// and glam += gy_t Re(c sl_t), gtheta += gy_t Re(c st_t) accumulate online.
// Per step (h, sl, st) -> a_t (I + N_t)(h, sl, st) + (u_t, 0, 0) with N_t
// nonzero only in its first column and N_t N_s = 0, so a segment's map is
// P (I + sum N) with P = prod a and sum N = (r-sum / lambda, i phi-sum):
// segments compose from (P, sum r, sum phi, local state).  Layout as the
// forward: one wave per (batch, head, segment), lane = mode, fp64 state.
// ---------------------------------------------------------------------------
// Triples (h, sl, st) are stored as three planes of complex values, so a wave's
// 64 modes move as contiguous 1 KB rows.
template <typename T, bool SUMMARY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void cplx_rtrl_kernel(RtrlParams p) {
    const int wave = threadIdx.x >> 6;
    const int unit = blockIdx.x * 4 + wave;
    if (unit >= p.B * p.H * p.G) return;
    const int s = unit / p.G, g = unit - s * p.G;
    const int b = s / p.H, hh = s - b * p.H;
    const int m = threadIdx.x & 63;
    const bool act = m < p.M;
    const int mc = act ? m : p.M - 1;
    const int L = p.L, M = p.M;
    const double lamd = p.lam[(int64_t)hh * p.slam + mc];
    const double lnl = log(lamd), ilam = 1.0 / lamd;
    const float th = p.theta[(int64_t)hh * p.stheta + mc];
    const int64_t pc = (int64_t)hh * p.sc + mc;
    const double c_re = p.c[2 * pc], c_im = p.c[2 * pc + 1];
    const float thmax = wave_absmax(th);
    const size_t us = ((size_t)s * p.G + g) * M + mc;   // (B*H, G, M)
    cd h = {0.0, 0.0}, sl = {0.0, 0.0}, stt = {0.0, 0.0}, P = {1.0, 0.0};
    double rsum = 0.0, psum = 0.0, gl = 0.0, gt = 0.0;
    if (!SUMMARY) {
        if (p.G > 1) {
            const size_t n3 = (size_t)p.B * p.H * p.G * M;
            h = ld_cd(p.carry, us);
            sl = ld_cd(p.carry, n3 + us);
            stt = ld_cd(p.carry, 2 * n3 + us);
        } else if (p.h0) {
            h = {p.h0[2 * ((size_t)s * M + mc)], p.h0[2 * ((size_t)s * M + mc) + 1]};
        }
        if (!act) h = sl = stt = cd{0.0, 0.0};
    }
    const int c0 = g * p.chunks_per_seg;
    const int c1 = min(c0 + p.chunks_per_seg, p.nchunks);
    const T* urow = (const T*)p.u + 2 * ((int64_t)b * p.su[0] + (int64_t)hh * p.su[1]);
    const T* rrow = (const T*)p.r + ((int64_t)b * p.sr[0] + (int64_t)hh * p.sr[1]);
    const T* prow = (const T*)p.phi + ((int64_t)b * p.sphi[0] + (int64_t)hh * p.sphi[1]);
    for (int ch = c0; ch < c1; ++ch) {
        const int t0 = ch * kCChunk;
        const int tl = t0 + (m & 31);
        const bool tv = tl < L;
        const float rv = tv ? to_f32(rrow[tl]) : 0.0f;
        const float pv = tv ? to_f32(prow[tl]) : 0.0f;
        const float gv = (!SUMMARY && tv) ? to_f32(((const T*)p.gy)[(size_t)s * L + tl]) : 0.0f;
        float yp[kCChunk];
        cplx_chunk(pv, thmax, t0 + kCChunk <= L, [&](auto fastc, auto fullc) {
            constexpr bool FAST = decltype(fastc)::value, FULL = decltype(fullc)::value;
#pragma unroll
            for (int hb = 0; hb < kCChunk / 16; ++hb) {
                float2 uv[16];
                load_u<T, 16>(urow, t0 + 16 * hb, L, p.su[2], mc, act, uv);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int j = 16 * hb + jj;
                    yp[j] = 0.0f;
                    if (FULL || t0 + j < L) {  // uniform
                        const float rj = lanev(rv, j), pj = lanev(pv, j);
                        const cd a = trans_a<FAST>(rj, lnl, pj, th);
                        const cd ah = cmul(a, h);
                        const double rl = (double)rj * ilam, ph = (double)pj;
                        sl = cfma(a, sl, cd{rl * ah.re, rl * ah.im});
                        stt = cfma(a, stt, cd{-ph * ah.im, ph * ah.re});
                        h = {ah.re + uv[jj].x, ah.im + uv[jj].y};
                        if (SUMMARY) {
                            P = cmul(a, P);
                            rsum += (double)rj;
                            psum += ph;
                        } else {
                            const double gj = lanev(gv, j);
                            gl = fma(gj, fma(c_re, sl.re, -c_im * sl.im), gl);
                            gt = fma(gj, fma(c_re, stt.re, -c_im * stt.im), gt);
                            yp[j] = (float)fma(c_re, h.re, -c_im * h.im);
                        }
                    }
                }
            }
        });
        if (!SUMMARY && p.y) {
            const float ys = wave_transpose_sum32(yp);
            const int t = t0 + (m >> 1);
            if ((m & 1) == 0 && t < L) ((T*)p.y)[(size_t)s * L + t] = from_f32<T>(ys);
        }
    }
    if (SUMMARY) {
        if (act) {
            const size_t n3 = (size_t)p.B * p.H * p.G * M;
            st_cd(p.segS, us, h);
            st_cd(p.segS, n3 + us, sl);
            st_cd(p.segS, 2 * n3 + us, stt);
            st_cd(p.segP, us, P);
        }
        if (m == 0) {
            p.segRP[2 * ((size_t)s * p.G + g)] = rsum;
            p.segRP[2 * ((size_t)s * p.G + g) + 1] = psum;
        }
        return;
    }
    if (!act) return;
    if (p.gh_last && g == p.G - 1) {   // <gh_last, h_{L-1}> in the real-pair convention
        const double gre = p.gh_last[2 * ((size_t)s * M + m)], gim = p.gh_last[2 * ((size_t)s * M + m) + 1];
        gl = fma(gre, sl.re, fma(gim, sl.im, gl));
        gt = fma(gre, stt.re, fma(gim, stt.im, gt));
    }
    const size_t po = (((size_t)b * p.G + g) * p.H + hh) * M + m;
    p.partL[po] = gl;
    p.partT[po] = gt;
}

// Entering (h, sl, st) of every segment, one lane per (batch, head, mode).
__global__ __launch_bounds__(256) void cplx_rtrl_combine_kernel(RtrlParams p) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= p.B * p.H * p.M) return;
    const int s = i / p.M, m = i - s * p.M;
    const double ilam = 1.0 / (double)p.lam[(int64_t)(s % p.H) * p.slam + m];
    const size_t n3 = (size_t)p.B * p.H * p.G * p.M;
    cd h = {0.0, 0.0}, sl = {0.0, 0.0}, stt = {0.0, 0.0};
    if (p.h0) h = {p.h0[2 * (size_t)i], p.h0[2 * (size_t)i + 1]};
    const size_t o0 = (size_t)s * p.G * p.M + m;
    const size_t r0 = (size_t)s * p.G;
    for (int g0 = 0; g0 < p.G; g0 += kCombBatch) {
        cd P[kCombBatch], S0[kCombBatch], S1[kCombBatch], S2[kCombBatch];
        double R[kCombBatch], Ph[kCombBatch];
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g0 + j < p.G) {
                const size_t o = o0 + (size_t)(g0 + j) * p.M;
                P[j] = ld_cd(p.segP, o);
                S0[j] = ld_cd(p.segS, o);
                S1[j] = ld_cd(p.segS, n3 + o);
                S2[j] = ld_cd(p.segS, 2 * n3 + o);
                R[j] = p.segRP[2 * (r0 + g0 + j)] * ilam;
                Ph[j] = p.segRP[2 * (r0 + g0 + j) + 1];
            }
#pragma unroll
        for (int j = 0; j < kCombBatch; ++j)
            if (g0 + j < p.G) {
                const size_t o = o0 + (size_t)(g0 + j) * p.M;
                st_cd(p.carry, o, h);
                st_cd(p.carry, n3 + o, sl);
                st_cd(p.carry, 2 * n3 + o, stt);
                const cd sl_in = {fma(R[j], h.re, sl.re), fma(R[j], h.im, sl.im)};
                const cd st_in = {fma(-Ph[j], h.im, stt.re), fma(Ph[j], h.re, stt.im)};
                sl = cfma(P[j], sl_in, S1[j]);
                stt = cfma(P[j], st_in, S2[j]);
                h = cfma(P[j], h, S0[j]);
            }
    }
}

// (B, G, H, M) partials -> glam, gtheta (H, M), one wave per (head, mode).
__global__ __launch_bounds__(256) void cplx_rtrl_reduce_kernel(RtrlParams p) {
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int HM = p.H * p.M;
    if (i >= HM) return;
    const int lane = threadIdx.x & 63;
    double sl = 0.0, st = 0.0;
    for (int k = lane; k < p.B * p.G; k += 64) {
        sl += p.partL[(size_t)k * HM + i];
        st += p.partT[(size_t)k * HM + i];
    }
    sl = wave_sum_f64(sl);
    st = wave_sum_f64(st);
    if (lane != 0) return;
    if (p.glam) p.glam[i] = (float)sl;
    if (p.gtheta) p.gtheta[i] = (float)st;
}

hipError_t launch_cplx_rtrl(const RtrlParams& p, bool summary, hipStream_t st) {
    const int units = p.B * p.H * p.G;
    if (p.dtype == 0) {
        if (summary) cplx_rtrl_kernel<float, true><<<(units + 3) / 4, 256, 0, st>>>(p);
        else cplx_rtrl_kernel<float, false><<<(units + 3) / 4, 256, 0, st>>>(p);
    } else {
        if (summary) cplx_rtrl_kernel<bf16_t, true><<<(units + 3) / 4, 256, 0, st>>>(p);
        else cplx_rtrl_kernel<bf16_t, false><<<(units + 3) / 4, 256, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_cplx_rtrl_combine(const RtrlParams& p, hipStream_t st) {
    const int n = p.B * p.H * p.M;
    cplx_rtrl_combine_kernel<<<(n + 255) / 256, 256, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_cplx_rtrl_reduce(const RtrlParams& p, hipStream_t st) {
    const int HM = p.H * p.M;
    cplx_rtrl_reduce_kernel<<<(HM + 3) / 4, 256, 0, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_cplx_fwd(const CplxParams& p, bool summary, hipStream_t st) {
    const int units = p.B * p.H * p.G;
    dim3 grid((units + 3) / 4), block(256);
    if (p.a) {  // given transitions: complex64 streams only
        if (p.dtype != 0) return hipErrorInvalidValue;
        if (summary) cplx_fwd_kernel<float, true, true><<<grid, block, 0, st>>>(p);
        else cplx_fwd_kernel<float, false, true><<<grid, block, 0, st>>>(p);
    } else if (p.dtype == 0) {
        if (summary) cplx_fwd_kernel<float, true><<<grid, block, 0, st>>>(p);
        else cplx_fwd_kernel<float, false><<<grid, block, 0, st>>>(p);
    } else {
        if (summary) cplx_fwd_kernel<bf16_t, true><<<grid, block, 0, st>>>(p);
        else cplx_fwd_kernel<bf16_t, false><<<grid, block, 0, st>>>(p);
    }
    return hipGetLastError();
}
hipError_t launch_cplx_bwd(const CplxParams& p, bool summary, hipStream_t st) {
    const int units = p.B * p.H * p.G;
    dim3 grid((units + 3) / 4), block(256);
    if (p.a) {
        if (p.dtype != 0) return hipErrorInvalidValue;
        if (summary) cplx_bwd_kernel<float, true, true><<<grid, block, 0, st>>>(p);
        else cplx_bwd_kernel<float, false, true><<<grid, block, 0, st>>>(p);
    } else if (p.dtype == 0) {
        if (summary) cplx_bwd_kernel<float, true><<<grid, block, 0, st>>>(p);
        else cplx_bwd_kernel<float, false><<<grid, block, 0, st>>>(p);
    } else {
        if (summary) cplx_bwd_kernel<bf16_t, true><<<grid, block, 0, st>>>(p);
        else cplx_bwd_kernel<bf16_t, false><<<grid, block, 0, st>>>(p);
    }
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
