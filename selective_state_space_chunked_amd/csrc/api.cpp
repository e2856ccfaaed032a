// Host side of the C ABI declared in include/ssmscan.h: argument validation
// (host-only, nothing touches the device before it passes), planning (chunk
// geometry, number of segments that run in parallel along the sequence),
// workspace layout and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ssmscan.h"
#include "kernels.hpp"

using namespace ssm;

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return code;
}
int ok() {
    g_detail.clear();
    return SSM_OK;
}

// Parallelism target: enough 256-lane workgroups to give every SIMD of the
// 256 compute units several waves.
constexpr int64_t kTargetWG = 1024;
constexpr size_t kAlign = 256;

struct Range {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlaps(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    auto a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}
// every output against every other buffer
int check_overlaps(const std::vector<Range>& ins, const std::vector<Range>& outs) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (const auto& r : ins)
            if (overlaps(outs[i], r)) return fail(SSM_ERR_LAYOUT, "output %s overlaps input %s", outs[i].name, r.name);
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(SSM_ERR_LAYOUT, "output %s overlaps output %s", outs[i].name, outs[j].name);
    }
    return SSM_OK;
}
int check_align(const void* p, size_t a, const char* name) {
    if (p && ((uintptr_t)p % a) != 0) return fail(SSM_ERR_LAYOUT, "%s is not %zu-byte aligned", name, a);
    return SSM_OK;
}
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p % 16) == 0; }

// bump allocator over the caller's workspace (or a size-only dry run)
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base((char*)b) {}
    template <typename T>
    T* take(size_t count) {
        off = (off + kAlign - 1) / kAlign * kAlign;
        T* p = base ? (T*)(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool is_complex(int mode) { return mode == SSM_COMPLEX_SHARED || mode == SSM_COMPLEX_DENSE; }

int device_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SSM_ERR_DEVICE, "%s: %s", what, hipGetErrorName(e));
    return SSM_OK;
}
// Optional per-kernel timing (ssm_profile_begin / ssm_profile_end).
struct Profile {
    bool on = false;
    int cap = 0, n = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch
    std::vector<const char*> names;
};
thread_local Profile g_prof;

void prof_pre(hipStream_t st) {
    if (g_prof.on && g_prof.n < g_prof.cap) hipEventRecord(g_prof.ev[2 * g_prof.n], st);
}
void prof_post(hipStream_t st, const char* what) {
    if (g_prof.on && g_prof.n < g_prof.cap) {
        hipEventRecord(g_prof.ev[2 * g_prof.n + 1], st);
        g_prof.names[g_prof.n] = what;
        ++g_prof.n;
    }
}

#define SSM_LAUNCH(expr, what)                            \
    do {                                                  \
        prof_pre(st);                                     \
        int rc_ = device_status((expr), what);            \
        if (rc_ != SSM_OK) return rc_;                    \
        prof_post(st, what);                              \
    } while (0)

// segment count along the sequence so the grid reaches the parallelism target
void plan_segments(int64_t wg_per_seg, int64_t nunits, int* G, int* per_seg, int64_t target = kTargetWG) {
    int64_t g = std::max<int64_t>(1, cdiv(target, std::max<int64_t>(1, wg_per_seg)));
    g = std::min<int64_t>(g, nunits);
    int64_t ps = cdiv(nunits, g);
    *per_seg = (int)ps;
    *G = (int)cdiv(nunits, ps);
}

// ---------------------------------------------------------------------------
// diagonal real / complex scans: shared validation
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// strided views (ssm_layout): per role, the logical shape, the dense strides
// and the strides this call uses
// ---------------------------------------------------------------------------
const char* const kRoleName[SSM_V_COUNT] = {"delta", "x", "A", "Bm", "C", "y", "gy", "gdelta", "gx", "r",
                                            "phi", "u", "lam", "theta", "c", "logits", "d", "b", "C", "dict"};
struct Views {
    int rank[SSM_V_COUNT] = {};
    int64_t dim[SSM_V_COUNT][4] = {};
    int64_t s[SSM_V_COUNT][4] = {};    // strides in use (dense unless given)
    bool given[SSM_V_COUNT] = {};
    void spec(int r, std::initializer_list<int64_t> dims, std::initializer_list<int64_t> dense) {
        rank[r] = (int)dims.size();
        int i = 0;
        for (int64_t d : dims) dim[r][i++] = d;
        i = 0;
        for (int64_t d : dense) s[r][i++] = d;
    }
    // elements spanned: 1 + sum (dim - 1) * stride (0 when a dimension is empty)
    size_t extent(int r) const {
        size_t e = 1;
        for (int i = 0; i < rank[r]; ++i) {
            if (dim[r][i] == 0) return 0;
            e += (size_t)(dim[r][i] - 1) * (size_t)s[r][i];
        }
        return e;
    }
    // element offsets of a stream row (b, c): b * s0 + c * s1
    int64_t sb(int r) const { return s[r][0]; }
    int64_t sd(int r) const { return s[r][1]; }
};

// An output's strides must give distinct elements: ordered by stride, every
// dimension of more than one element strides past everything inside it.
bool distinct_elements(const Views& v, int r) {
    int idx[4];
    int n = 0;
    for (int i = 0; i < v.rank[r]; ++i)
        if (v.dim[r][i] > 1) idx[n++] = i;
    std::sort(idx, idx + n, [&](int x, int y) { return v.s[r][x] < v.s[r][y]; });
    int64_t span = 1;
    for (int k = 0; k < n; ++k) {
        const int i = idx[k];
        if (v.s[r][i] < span) return false;
        span = v.s[r][i] * (v.dim[r][i] - 1) + span;
    }
    return true;
}

// Take the caller's strides for the roles in `use_in` (inputs) and `use_out`
// (outputs); any other given role is refused.
int resolve_views(const ssm_layout* lay, uint64_t use_in, uint64_t use_out, Views* v, const char* who) {
    if (!lay) return SSM_OK;
    if (lay->given >> SSM_V_COUNT) return fail(SSM_ERR_UNSUPPORTED, "layout names an unknown role");
    for (int r = 0; r < SSM_V_COUNT; ++r) {
        if (!((lay->given >> r) & 1)) continue;
        const bool in = (use_in >> r) & 1, out = (use_out >> r) & 1;
        if (!in && !out) return fail(SSM_ERR_UNSUPPORTED, "%s does not take %s as a strided view", who, kRoleName[r]);
        const int k = v->rank[r];
        for (int i = 0; i < k; ++i) {
            const int64_t st = lay->stride[r][i];
            if (st < 0) return fail(SSM_ERR_LAYOUT, "%s: negative stride %lld", kRoleName[r], (long long)st);
            v->s[r][i] = st;
        }
        // the innermost dimension must be contiguous (its stride is irrelevant for a single element);
        // a rank-1 role (the per-head A) is indexed with its stride, which may be 0 on an input
        if (k > 1 || out) {
            if (v->dim[r][k - 1] > 1 && v->s[r][k - 1] != 1)
                return fail(SSM_ERR_LAYOUT, "%s: innermost stride must be 1 (got %lld)", kRoleName[r],
                            (long long)v->s[r][k - 1]);
            v->s[r][k - 1] = 1;
        }
        if (out && !distinct_elements(*v, r))
            return fail(SSM_ERR_LAYOUT, "output %s: strides must give distinct elements (no stride 0)", kRoleName[r]);
        if (v->s[r][0] >= (1LL << 40) || (k > 1 && v->s[r][1] >= (1LL << 40)))
            return fail(SSM_ERR_LAYOUT, "%s: stride too large", kRoleName[r]);
        v->given[r] = true;
    }
    return SSM_OK;
}
constexpr uint64_t bit(int r) { return 1ull << r; }

// Entry points, for the roles each takes as views.
enum Entry { E_FWD, E_BWD, E_SENS, E_RTRL };

struct ScanPlan {
    int mode, dtype;
    int64_t B, D, L, N;
    int T;         // checkpoint interval
    int kpl;       // selective: steps per lane (T/16)
    int nchunks;   // ceil(L/T)
    size_t esz;    // bytes per streamed element
    bool empty;    // no batch rows, channels or steps: only h_last / gh0 / parameter gradients are defined
    int disc;      // SSM_EULER or SSM_ZOH
    bool perd;     // selective: Bm and C given per channel
    int64_t P, H;  // SSM_HEAD_SCALAR: channels per head, heads
    Views v;
};

void scan_view_specs(ScanPlan* pl) {
    const int64_t B = pl->B, D = pl->D, L = pl->L, N = pl->N;
    Views& v = pl->v;
    for (int r : {SSM_V_DELTA, SSM_V_X, SSM_V_Y, SSM_V_GY, SSM_V_GDELTA, SSM_V_GX, SSM_V_R, SSM_V_PHI})
        v.spec(r, {B, D, L}, {D * L, L, 1});
    v.spec(SSM_V_A, {D, N}, {N, 1});
    v.spec(SSM_V_BM, {B, D, L, N}, {L * N, 0, N, 1});   // shared by the channels
    v.spec(SSM_V_C, {B, D, L, N}, {L * N, 0, N, 1});
    v.spec(SSM_V_U, {B, D, L, N}, {D * L * N, L * N, N, 1});
    for (int r : {SSM_V_LAM, SSM_V_THETA, SSM_V_CC}) v.spec(r, {D, N}, {N, 1});
    if (pl->mode == SSM_HEAD_SCALAR) {   // per-head step sizes and transitions
        const int64_t H = pl->H;
        for (int r : {SSM_V_DELTA, SSM_V_GDELTA}) v.spec(r, {B, H, L}, {H * L, L, 1});
        v.spec(SSM_V_A, {H}, {1});
    }
}

// sel_default_T: the selective mode's checkpoint interval when chunk_len is 0
int validate_scan_args(const ssm_scan_args* a, ScanPlan* pl, int sel_default_T = 256, Entry entry = E_FWD) {
    if (!a) return fail(SSM_ERR_NULL, "args is NULL");
    pl->mode = a->mode;
    pl->dtype = a->dtype;
    pl->B = a->batch; pl->D = a->channels; pl->L = a->length; pl->N = a->state;
    if (a->mode != SSM_REAL_SELECTIVE && a->mode != SSM_REAL_DENSE && a->mode != SSM_COMPLEX_SHARED &&
        a->mode != SSM_COMPLEX_DENSE && a->mode != SSM_HEAD_SCALAR)
        return fail(SSM_ERR_UNSUPPORTED, "unknown mode %d", a->mode);
    if (a->dtype != SSM_F32 && a->dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "unknown dtype %d", a->dtype);
    pl->P = 0;
    pl->H = 0;
    if (a->mode == SSM_HEAD_SCALAR) {
        if (a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 48 && a->head_dim != 64)
            return fail(SSM_ERR_UNSUPPORTED, "head_dim %lld not supported (16, 32, 48 or 64)", (long long)a->head_dim);
        if (a->channels % a->head_dim)
            return fail(SSM_ERR_SHAPE, "channels %lld are not a multiple of head_dim %lld", (long long)a->channels,
                        (long long)a->head_dim);
        if (a->state != 16 && a->state != 32 && a->state != 48 && a->state != 64)
            return fail(SSM_ERR_UNSUPPORTED, "SSM_HEAD_SCALAR takes state 16, 32, 48 or 64 (got %lld)",
                        (long long)a->state);
        if (entry != E_FWD && entry != E_BWD)
            return fail(SSM_ERR_UNSUPPORTED, "SSM_HEAD_SCALAR supports ssm_scan_fwd and ssm_scan_bwd");
        pl->P = a->head_dim;
        pl->H = a->channels / a->head_dim;
    } else if (a->head_dim != 0) {
        return fail(SSM_ERR_SHAPE, "head_dim applies to SSM_HEAD_SCALAR only");
    }
    if (a->dtype == SSM_BF16 && (a->mode == SSM_REAL_DENSE || a->mode == SSM_COMPLEX_DENSE))
        return fail(SSM_ERR_DTYPE, "bf16 streams are supported by SSM_REAL_SELECTIVE, SSM_COMPLEX_SHARED and "
                                   "SSM_HEAD_SCALAR only");
    if (pl->B < 0 || pl->D < 0 || pl->L < 0 || pl->N < 1)
        return fail(SSM_ERR_SHAPE, "sizes must be >= 0 and state >= 1 (B=%lld D=%lld L=%lld N=%lld)",
                    (long long)pl->B, (long long)pl->D, (long long)pl->L, (long long)pl->N);
    pl->empty = pl->B == 0 || pl->D == 0 || pl->L == 0;
    const int64_t nmax = is_complex(a->mode) || a->mode == SSM_HEAD_SCALAR ? 64 : 16;
    if (pl->N > nmax) return fail(SSM_ERR_SHAPE, "state size %lld exceeds %lld", (long long)pl->N, (long long)nmax);
    if (pl->B > 65535) return fail(SSM_ERR_SHAPE, "batch %lld exceeds 65535", (long long)pl->B);
    if (pl->L >= (1LL << 31) || pl->D >= (1LL << 24) || pl->B * pl->D * pl->L * pl->N >= (1LL << 46))
        return fail(SSM_ERR_SHAPE, "problem too large");
    pl->esz = a->dtype == SSM_BF16 ? 2 : 4;
    int T = (int)a->chunk_len;
    if (a->mode == SSM_REAL_SELECTIVE) {
        if (T == 0) T = sel_default_T;
        if (T != 64 && T != 128 && T != 256)
            return fail(SSM_ERR_UNSUPPORTED, "chunk_len %d not supported (64, 128 or 256)", T);
        pl->kpl = T / 16;
    } else if (a->mode == SSM_HEAD_SCALAR) {
        if (T == 0) T = 64;
        if (T != 64) return fail(SSM_ERR_UNSUPPORTED, "chunk_len %d not supported (64)", T);
        pl->kpl = 4;   // the backward's tiles (16 lanes x 4 steps)
    } else {
        if (T == 0) T = 32;
        if (T != 32) return fail(SSM_ERR_UNSUPPORTED, "chunk_len %d not supported (32)", T);
        pl->kpl = 0;
    }
    if (a->chunk_len < 0) return fail(SSM_ERR_SHAPE, "negative chunk_len");
    pl->T = T;
    pl->nchunks = (int)cdiv(pl->L, T);
    const size_t BDL = pl->B * pl->D * pl->L;
    const size_t BLN = pl->B * pl->L * pl->N;
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSM_ERR_SHAPE, "delta_softplus must be 0 or 1 (got %d)", a->delta_softplus);
    if (a->mode != SSM_REAL_SELECTIVE && (a->delta_bias || a->delta_softplus))
        return fail(SSM_ERR_UNSUPPORTED, "delta_bias / delta_softplus apply to SSM_REAL_SELECTIVE only");
    if (a->discretization != SSM_EULER && a->discretization != SSM_ZOH)
        return fail(SSM_ERR_SHAPE, "unknown discretization %d", a->discretization);
    pl->disc = a->discretization;
    if (pl->disc == SSM_ZOH && a->mode != SSM_REAL_SELECTIVE)
        return fail(SSM_ERR_UNSUPPORTED, "the ZOH discretisation applies to SSM_REAL_SELECTIVE only");
    if (pl->disc == SSM_ZOH && entry != E_FWD && entry != E_BWD)
        return fail(SSM_ERR_UNSUPPORTED, "the sensitivity entry points take the Euler discretisation only");
    scan_view_specs(pl);
    {
        uint64_t in = 0, out = 0;
        if (a->mode == SSM_REAL_SELECTIVE || a->mode == SSM_HEAD_SCALAR) {
            in = bit(SSM_V_DELTA) | bit(SSM_V_X) | bit(SSM_V_A) | bit(SSM_V_BM) | bit(SSM_V_C);
            if (entry == E_FWD) out = bit(SSM_V_Y);
            if (entry == E_BWD) { in |= bit(SSM_V_GY); out = bit(SSM_V_GDELTA) | bit(SSM_V_GX); }
        } else if (a->mode == SSM_COMPLEX_SHARED) {
            in = bit(SSM_V_R) | bit(SSM_V_PHI) | bit(SSM_V_U) | bit(SSM_V_LAM) | bit(SSM_V_THETA) | bit(SSM_V_CC);
        }
        if (int rc = resolve_views(a->layout, in, out, &pl->v, "this mode and entry point")) return rc;
    }
    pl->perd = false;
    if (a->mode == SSM_REAL_SELECTIVE) {
        // either one per channel: both are read per channel (a shared one through its zero channel
        // stride) and both gradients are per channel
        pl->perd = pl->D > 1 && (pl->v.sd(SSM_V_BM) != 0 || pl->v.sd(SSM_V_C) != 0);
        if (pl->perd && entry != E_FWD && entry != E_BWD)
            return fail(SSM_ERR_UNSUPPORTED, "the sensitivity entry points take Bm and C shared by the channels");
        if (pl->perd && pl->disc == SSM_ZOH)
            return fail(SSM_ERR_UNSUPPORTED, "the ZOH discretisation takes Bm and C shared by the channels");
    }
    if (a->mode == SSM_HEAD_SCALAR) {
        if (pl->D > 1 && (pl->v.sd(SSM_V_BM) != 0 || pl->v.sd(SSM_V_C) != 0))
            return fail(SSM_ERR_UNSUPPORTED, "SSM_HEAD_SCALAR takes Bm and C shared by the channels");
        if (!pl->empty && (!a->delta || !a->x || !a->A || !a->Bm || !a->C))
            return fail(SSM_ERR_NULL, "SSM_HEAD_SCALAR needs delta, x, A, Bm and C");
        int rc;
        const size_t al = pl->esz;
        if ((rc = check_align(a->delta, al, "delta")) || (rc = check_align(a->x, al, "x")) ||
            (rc = check_align(a->Bm, al, "Bm")) || (rc = check_align(a->C, al, "C")) ||
            (rc = check_align(a->A, 4, "A")) || (rc = check_align(a->h0, 4, "h0")))
            return rc;
        return SSM_OK;
    }
    if (a->mode == SSM_REAL_SELECTIVE) {
        if (!pl->empty && (!a->delta || !a->x || !a->A || !a->Bm || !a->C))
            return fail(SSM_ERR_NULL, "SSM_REAL_SELECTIVE needs delta, x, A, Bm and C");
        if (int rc = check_align(a->delta_bias, 4, "delta_bias")) return rc;
        const size_t al = pl->esz;
        int rc;
        if ((rc = check_align(a->delta, al, "delta")) || (rc = check_align(a->x, al, "x")) ||
            (rc = check_align(a->Bm, al, "Bm")) || (rc = check_align(a->C, al, "C")) ||
            (rc = check_align(a->A, 4, "A")) || (rc = check_align(a->h0, 4, "h0")))
            return rc;
        (void)BDL; (void)BLN;
    } else if (a->mode == SSM_REAL_DENSE) {
        if (!pl->empty && (!a->a || !a->b || !a->C)) return fail(SSM_ERR_NULL, "SSM_REAL_DENSE needs a, b and C");
        int rc;
        if ((rc = check_align(a->a, 4, "a")) || (rc = check_align(a->b, 4, "b")) ||
            (rc = check_align(a->C, 4, "C")) || (rc = check_align(a->h0, 4, "h0")))
            return rc;
    } else if (a->mode == SSM_COMPLEX_DENSE) {
        if (!pl->empty && (!a->a || !a->u || !a->c)) return fail(SSM_ERR_NULL, "SSM_COMPLEX_DENSE needs a, u and c");
        int rc;
        if ((rc = check_align(a->a, 8, "a")) || (rc = check_align(a->u, 8, "u")) || (rc = check_align(a->c, 8, "c")) ||
            (rc = check_align(a->h0, 8, "h0")))
            return rc;
    } else {
        if (!pl->empty && (!a->r || !a->phi || !a->lam || !a->theta || !a->u || !a->c))
            return fail(SSM_ERR_NULL, "SSM_COMPLEX_SHARED needs r, phi, lam, theta, u and c");
        int rc;
        if ((rc = check_align(a->u, 2 * pl->esz, "u")) || (rc = check_align(a->c, 8, "c")) ||
            (rc = check_align(a->r, pl->esz, "r")) || (rc = check_align(a->phi, pl->esz, "phi")) ||
            (rc = check_align(a->h0, 8, "h0")))
            return rc;
    }
    return SSM_OK;
}

std::vector<Range> scan_inputs(const ssm_scan_args* a, const ScanPlan& p) {
    const size_t BDL = p.B * p.D * p.L, BDLN = BDL * p.N;
    const size_t st = p.N * (is_complex(p.mode) ? 8 : 4);
    const Views& v = p.v;
    return {
        {a->delta, v.extent(SSM_V_DELTA) * p.esz, "delta"}, {a->x, v.extent(SSM_V_X) * p.esz, "x"},
        {a->A, v.extent(SSM_V_A) * 4, "A"}, {a->Bm, v.extent(SSM_V_BM) * p.esz, "Bm"},
        {a->a, BDLN * (p.mode == SSM_COMPLEX_DENSE ? 8 : 4), "a"}, {a->b, BDLN * 4, "b"},
        {a->C, v.extent(SSM_V_C) * (p.mode == SSM_REAL_DENSE ? 4 : p.esz), "C"},
        {a->r, v.extent(SSM_V_R) * p.esz, "r"}, {a->phi, v.extent(SSM_V_PHI) * p.esz, "phi"},
        {a->lam, v.extent(SSM_V_LAM) * 4, "lam"}, {a->theta, v.extent(SSM_V_THETA) * 4, "theta"},
        {a->u, v.extent(SSM_V_U) * 2 * p.esz, "u"}, {a->c, v.extent(SSM_V_CC) * 8, "c"},
        {a->h0, (size_t)p.B * p.D * st, "h0"},
        {a->delta_bias, (size_t)p.D * 4, "delta_bias"},
    };
}

// ---------------------------------------------------------------------------
// selective: forward plan + workspace
// ---------------------------------------------------------------------------
struct SelFwdLayout {
    int G, tps;
    float *segP = nullptr, *segS = nullptr, *carry = nullptr;
};
void sel_fwd_layout(const ScanPlan& p, Carve& cv, SelFwdLayout* lay) {
    const int64_t wg = cdiv(p.D, 16) * p.B;
    plan_segments(wg, p.nchunks, &lay->G, &lay->tps);
    if (lay->G > 1) {
        const size_t n = (size_t)p.B * p.D * lay->G * p.N;
        lay->segP = cv.take<float>(n);
        lay->segS = cv.take<float>(n);
        lay->carry = cv.take<float>(n);
    }
}

// 16-byte loads and stores of the (B,D,L) streams: every row start aligned
// (steps contiguous, batch and channel strides whole 16-byte units)
int sel_vec(const ScanPlan& p, std::initializer_list<const void*> ptrs, std::initializer_list<int> roles = {}) {
    if (p.L % 8 != 0) return 0;
    for (const void* q : ptrs)
        if (!aligned16(q)) return 0;
    const int64_t unit = 16 / (int64_t)p.esz;
    for (int r : roles)
        if (p.v.s[r][0] % unit || p.v.s[r][1] % unit) return 0;
    return 1;
}
// 16-byte loads of B_t / C_t rows (state dimension contiguous)
int sel_bc_vec(const ScanPlan& p, const void* Bm, const void* C) {
    const int64_t unit = 16 / (int64_t)p.esz;
    if (!aligned16(Bm) || !aligned16(C) || p.N % unit) return 0;
    for (int r : {SSM_V_BM, SSM_V_C})
        if (p.v.s[r][0] % unit || p.v.s[r][2] % unit) return 0;
    return 1;
}
template <int K>
void copy_strides(int64_t (&dst)[K], const ScanPlan& p, int r) {
    for (int i = 0; i < K; ++i) dst[i] = p.v.s[r][i];
}
int sel_var(const ScanPlan& p) { return p.perd ? kVarPerD : p.disc == SSM_ZOH ? kVarZoh : kVarEuler; }

// The impulse sensitivity formed by the main pass (N = 16, Euler, shared B_t and C_t, G > 1): the summary
// pass writes the tile sums of delta, the suffix kernel turns them into send, the main pass writes s.
struct FwdSens {
    void* s;         // nullable when s_delta is given
    void* s_delta;   // nullable: d y[t_out] / d delta
    double* send;
    int t_out;
};
int run_sel_fwd(const ssm_scan_args* a, const ScanPlan& p, const SelFwdLayout& lay, void* y, float* h_last,
                float* ckpt, float* tile_dsum, hipStream_t st, const FwdSens* sens = nullptr) {
    SelFwdParams q{};
    q.delta = a->delta; q.x = a->x; q.A = a->A; q.Bm = a->Bm; q.C = a->C; q.h0 = a->h0;
    q.carry_in = lay.carry;
    q.y = y; q.h_last = h_last; q.ckpt = ckpt; q.tile_dsum = tile_dsum;
    q.segP = lay.segP; q.segS = lay.segS;
    q.B = (int)p.B; q.D = (int)p.D; q.L = (int)p.L; q.N = (int)p.N;
    q.ntiles = p.nchunks; q.tiles_per_seg = lay.tps; q.G = lay.G;
    q.vec = sel_vec(p, {a->delta, a->x, y}, {SSM_V_DELTA, SSM_V_X, SSM_V_Y});
    q.stepf = StepXform{a->delta_bias, a->delta_softplus};
    copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sx, p, SSM_V_X); copy_strides(q.sy, p, SSM_V_Y);
    copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
    q.sA = p.v.s[SSM_V_A][0];
    q.bc_vec = sel_bc_vec(p, a->Bm, a->C);
    q.var = sel_var(p);
    if (sens) {
        q.vec = sel_vec(p, {a->delta, a->x, y, sens->s, sens->s_delta}, {SSM_V_DELTA, SSM_V_X, SSM_V_Y});
    }
    if (lay.G > 1) {
        SelFwdParams qs = q;
        qs.tile_dsum = sens ? tile_dsum : nullptr;   // with the sensitivity the main pass writes none
        SSM_LAUNCH(launch_sel_fwd(qs, p.dtype, p.kpl, true, st), "selective forward summary");
        SSM_LAUNCH(launch_seg_combine_fwd(lay.segP, lay.segS, a->h0, lay.carry, (int)(p.B * p.D), lay.G,
                                          (int)p.N, st), "segment combine");
    }
    if (sens) {
        SSM_LAUNCH(launch_sens_suffix(a->delta, p.v.s[SSM_V_DELTA][0], p.v.s[SSM_V_DELTA][1],
                                      StepXform{a->delta_bias, a->delta_softplus}, tile_dsum, sens->send, (int)p.B,
                                      (int)p.D, (int)p.L, p.nchunks, p.T, sens->t_out, p.dtype, st),
                   "suffix sums");
        q.tile_dsum = nullptr;
        q.s = sens->s; q.s_delta = sens->s_delta; q.send = sens->send; q.t_out = sens->t_out;
        SSM_LAUNCH(launch_sel_fwd_sens(q, p.dtype, p.kpl, st), "selective forward + sensitivity");
        return SSM_OK;
    }
    SSM_LAUNCH(launch_sel_fwd(q, p.dtype, p.kpl, false, st), "selective forward");
    return SSM_OK;
}

// ---------------------------------------------------------------------------
// selective: backward plan + workspace
// ---------------------------------------------------------------------------
struct SelBwdLayout {
    SelFwdLayout fwd;          // only when checkpoints are recomputed
    float* ckpt = nullptr;
    int G, tps;
    float *segQ = nullptr, *segR = nullptr, *nu = nullptr;
    float *partB = nullptr, *partC = nullptr, *partA = nullptr, *partBias = nullptr;
};
void sel_bwd_layout(const ScanPlan& p, bool have_ckpt, bool wantB, bool wantC, bool wantA, bool wantBias, Carve& cv,
                    SelBwdLayout* lay) {
    if (!have_ckpt) {
        lay->ckpt = cv.take<float>((size_t)p.B * p.D * p.nchunks * p.N);
        sel_fwd_layout(p, cv, &lay->fwd);
    }
    // 512-lane workgroups, one per compute unit at a time: two rounds of 256 CUs
    const int64_t wg = cdiv(p.D, sel_bwd_rows()) * p.B;
    plan_segments(wg, p.nchunks, &lay->G, &lay->tps, kTargetWG / 2);
    if (lay->G > 1) {
        const size_t n = (size_t)p.B * p.D * lay->G * p.N;
        lay->segQ = cv.take<float>(n);
        lay->segR = cv.take<float>(n);
        lay->nu = cv.take<float>(n);
    }
    const size_t np = (size_t)cdiv(p.D, sel_bwd_rows()) * p.B * p.N * p.L;
    if (wantB) lay->partB = cv.take<float>(np);
    if (wantC) lay->partC = cv.take<float>(np);
    if (wantA) lay->partA = cv.take<float>((size_t)p.B * lay->G * p.D * p.N);
    if (wantBias) lay->partBias = cv.take<float>((size_t)p.B * lay->G * p.D);
}

// ---------------------------------------------------------------------------
// scalar transition per head: the matrix-form forward
// ---------------------------------------------------------------------------
struct HeadFwdLayout {
    float *state = nullptr, *decay = nullptr;
};
void head_fwd_layout(const ScanPlan& p, Carve& cv, HeadFwdLayout* l) {
    l->state = cv.take<float>((size_t)p.B * p.H * p.nchunks * p.N * p.P);
    l->decay = cv.take<float>((size_t)p.B * p.H * p.nchunks);
}
// y nullable: only the entering states (checkpoints, h_last) are produced
int run_head_fwd(const ssm_scan_args* a, const ScanPlan& p, const HeadFwdLayout& l, void* y, float* h_last,
                 float* ckpt, hipStream_t st) {
    HeadParams q{};
    q.delta = a->delta; q.x = a->x; q.A = a->A; q.Bm = a->Bm; q.C = a->C; q.h0 = a->h0;
    copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sx, p, SSM_V_X); copy_strides(q.sy, p, SSM_V_Y);
    copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
    q.sA = p.v.s[SSM_V_A][0];
    q.y = y; q.h_last = h_last; q.ckpt = ckpt;
    q.state = l.state; q.decay = l.decay;
    q.B = (int)p.B; q.H = (int)p.H; q.P = (int)p.P; q.L = (int)p.L; q.N = (int)p.N; q.nchunks = p.nchunks;
    {   // 16-byte row loads need 16-byte aligned rows; 4-step stores of y, 4-element aligned rows
        const int64_t e16 = 16 / (int64_t)p.esz;
        auto al = [](const void* ptr, int64_t bytes) { return ((uintptr_t)ptr % (uintptr_t)bytes) == 0; };
        q.vx = al(a->x, 16) && q.sx[0] % e16 == 0 && q.sx[1] % e16 == 0;
        q.vb = al(a->Bm, 16) && q.sBm[0] % e16 == 0 && q.sBm[2] % e16 == 0;
        q.vc = al(a->C, 16) && q.sC[0] % e16 == 0 && q.sC[2] % e16 == 0;
        q.vy = y && al(y, 4 * (int64_t)p.esz) && q.sy[0] % 4 == 0 && q.sy[1] % 4 == 0;
    }
    SSM_LAUNCH(launch_head_state(q, p.dtype, st), "head chunk states (matrix cores)");
    SSM_LAUNCH(launch_head_chain(q, st), "head chunk chain");
    if (y) SSM_LAUNCH(launch_head_out(q, p.dtype, st), "head outputs (matrix cores)");
    return SSM_OK;
}

// ---------------------------------------------------------------------------
// entry-point helpers per mode (dense, complex and PD live further below)
// ---------------------------------------------------------------------------
int scan_fwd_impl(const ssm_scan_args* a, const ssm_scan_fwd_out* out, void* ws, size_t ws_bytes,
                  hipStream_t st, size_t* need_only);
int scan_bwd_impl(const ssm_scan_args* a, const ssm_scan_bwd_in* in, const ssm_scan_grads* g, void* ws,
                  size_t ws_bytes, hipStream_t st, size_t* need_only);
int impulse_impl(const ssm_scan_args* a, int64_t t_out, void* y, void* s, void* s_delta, bool with_delta,
                 void* ws, size_t ws_bytes, hipStream_t st, size_t* need_only);
int pd_fwd_impl(const pd_scan_args* a, const pd_scan_fwd_out* out, void* ws, size_t ws_bytes, hipStream_t st,
                size_t* need_only);
int pd_bwd_impl(const pd_scan_args* a, const pd_scan_bwd_in* in, const pd_scan_grads* g, void* ws,
                size_t ws_bytes, hipStream_t st, size_t* need_only);

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return SSM_OK;
    if (!ws) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (((uintptr_t)ws % kAlign) != 0) return fail(SSM_ERR_LAYOUT, "workspace is not %zu-byte aligned", kAlign);
    return SSM_OK;
}

// ======================= dense + complex declarations ======================
int dense_fwd(const ssm_scan_args* a, const ScanPlan& p, const ssm_scan_fwd_out* out, Carve& cv, bool dry,
              hipStream_t st);
int dense_bwd(const ssm_scan_args* a, const ScanPlan& p, const ssm_scan_bwd_in* in, const ssm_scan_grads* g,
              Carve& cv, bool dry, hipStream_t st);
int cplx_fwd(const ssm_scan_args* a, const ScanPlan& p, const ssm_scan_fwd_out* out, Carve& cv, bool dry,
             hipStream_t st);
int cplx_bwd(const ssm_scan_args* a, const ScanPlan& p, const ssm_scan_bwd_in* in, const ssm_scan_grads* g,
             Carve& cv, bool dry, hipStream_t st);

// ---------------------------------------------------------------------------
// ssm_scan_fwd
// ---------------------------------------------------------------------------
int scan_fwd_impl(const ssm_scan_args* a, const ssm_scan_fwd_out* out, void* ws, size_t ws_bytes,
                  hipStream_t st, size_t* need_only) {
    ScanPlan p;
    int rc = validate_scan_args(a, &p);
    if (rc) return rc;
    if (!need_only) {
        if (!out) return fail(SSM_ERR_NULL, "out is NULL");
        const size_t st_b = is_complex(p.mode) ? 8 : 4;
        const size_t yb = p.v.extent(SSM_V_Y) * (p.mode == SSM_REAL_DENSE ? 4 : p.esz);  // esz is 4 for complex dense
        const size_t hb = p.B * p.D * p.N * st_b;
        std::vector<Range> outs = {{out->y, yb, "y"}, {out->h_last, hb, "h_last"},
                                   {out->ckpt, hb * p.nchunks, "ckpt"}};
        if ((rc = check_align(out->y, p.mode == SSM_REAL_DENSE ? 4 : p.esz, "y")) ||
            (rc = check_align(out->h_last, st_b, "h_last")) || (rc = check_align(out->ckpt, st_b, "ckpt")))
            return rc;
        if ((rc = check_overlaps(scan_inputs(a, p), outs))) return rc;
    }
    if (p.empty) {   // y and the checkpoints have no elements; h_last = h0 (or 0)
        if (need_only) { *need_only = 0; return ok(); }
        const size_t nh = p.B * p.D * p.N * (is_complex(p.mode) ? 2 : 1);
        SSM_LAUNCH(launch_fill_copy_f32(out->h_last, a->h0, nh, st), "h_last of an empty scan");
        return ok();
    }
    Carve cv(nullptr);
    if (p.mode == SSM_HEAD_SCALAR) {
        HeadFwdLayout lay;
        head_fwd_layout(p, cv, &lay);
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        head_fwd_layout(p, real, &lay);
        if ((rc = run_head_fwd(a, p, lay, out->y, out->h_last, out->ckpt, st))) return rc;
        return ok();
    }
    if (p.mode == SSM_REAL_SELECTIVE) {
        SelFwdLayout lay;
        sel_fwd_layout(p, cv, &lay);
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        sel_fwd_layout(p, real, &lay);
        if ((rc = run_sel_fwd(a, p, lay, out->y, out->h_last, out->ckpt, nullptr, st))) return rc;
        return ok();
    }
    if (p.mode == SSM_REAL_DENSE) {
        if ((rc = dense_fwd(a, p, out, cv, true, st))) return rc;
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        if ((rc = dense_fwd(a, p, out, real, false, st))) return rc;
        return ok();
    }
    if ((rc = cplx_fwd(a, p, out, cv, true, st))) return rc;
    if (need_only) { *need_only = cv.off; return ok(); }
    if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
    Carve real(ws);
    if ((rc = cplx_fwd(a, p, out, real, false, st))) return rc;
    return ok();
}

// ---------------------------------------------------------------------------
// ssm_scan_bwd
// ---------------------------------------------------------------------------
int scan_bwd_impl(const ssm_scan_args* a, const ssm_scan_bwd_in* in, const ssm_scan_grads* g, void* ws,
                  size_t ws_bytes, hipStream_t st, size_t* need_only) {
    ScanPlan p;
    int rc = validate_scan_args(a, &p, 256, E_BWD);
    if (rc) return rc;
    static const ssm_scan_grads kNoGrads{};
    static const ssm_scan_bwd_in kNoIn{};
    if (!need_only) {
        if (!in) return fail(SSM_ERR_NULL, "in is NULL");
        if (!g) return fail(SSM_ERR_NULL, "grads is NULL");
        if (!in->gy && !p.empty) return fail(SSM_ERR_NULL, "gy is NULL");
    }
    if (!in) in = &kNoIn;
    if (!g) g = &kNoGrads;
    const bool have_ckpt = need_only ? false : in->ckpt != nullptr;
    if (!need_only) {
        const size_t st_b = is_complex(p.mode) ? 8 : 4;
        const size_t es = p.mode == SSM_REAL_DENSE ? 4 : p.esz;
        const size_t BDL = p.B * p.D * p.L, BLN = p.B * p.L * p.N;
        const size_t hb = p.B * p.D * p.N * st_b;
        std::vector<Range> ins = scan_inputs(a, p);
        ins.push_back({in->gy, p.v.extent(SSM_V_GY) * es, "gy"});
        ins.push_back({in->gh_last, hb, "gh_last"});
        ins.push_back({in->ckpt, hb * p.nchunks, "ckpt"});
        const size_t gbc = p.perd ? BDL * p.N : BLN;   // per-channel Bm / C: gradients per channel
        std::vector<Range> outs = {
            {g->gdelta, p.v.extent(SSM_V_GDELTA) * es, "gdelta"}, {g->gx, p.v.extent(SSM_V_GX) * es, "gx"},
            {g->gA, (p.mode == SSM_HEAD_SCALAR ? (size_t)p.H : (size_t)p.D * p.N) * 4, "gA"},
            {g->gBm, gbc * es, "gBm"}, {g->ga, BDL * p.N * (p.mode == SSM_COMPLEX_DENSE ? 8 : 4), "ga"},
            {g->gb, BDL * p.N * 4, "gb"},
            {g->gC, gbc * es, "gC"}, {g->gu, BDL * p.N * 2 * es, "gu"}, {g->gr, BDL * es, "gr"},
            {g->gphi, BDL * es, "gphi"}, {g->glam, (size_t)p.D * p.N * 4, "glam"},
            {g->gtheta, (size_t)p.D * p.N * 4, "gtheta"}, {g->gc, (size_t)p.D * p.N * 8, "gc"},
            {g->gh0, hb, "gh0"}, {g->gdelta_bias, (size_t)p.D * 4, "gdelta_bias"}};
        for (const auto& o : outs)
            if ((rc = check_align(o.p, 2, o.name))) return rc;
        if ((rc = check_overlaps(ins, outs))) return rc;
    }
    if (p.empty) {   // stream gradients have no elements; gh0 = gh_last (or 0), parameter gradients 0
        if (need_only) { *need_only = 0; return ok(); }
        const size_t cx = is_complex(p.mode) ? 2 : 1, dn = (size_t)p.D * p.N;
        SSM_LAUNCH(launch_fill_copy_f32(g->gh0, in->gh_last, p.B * p.D * p.N * cx, st), "gh0 of an empty scan");
        // gBm and gC sum over channels: with D = 0 but B, L > 0 they have elements, all zero
        const size_t btn = p.D == 0 ? p.B * p.L * p.N : 0;
        if (p.mode == SSM_HEAD_SCALAR) {
            SSM_LAUNCH(launch_fill_copy_f32(g->gA, nullptr, (size_t)p.H, st), "zero gA");
            SSM_LAUNCH(launch_zero_bytes(g->gBm, btn * p.esz, st), "zero gBm");
            SSM_LAUNCH(launch_zero_bytes(g->gC, btn * p.esz, st), "zero gC");
        } else if (p.mode == SSM_REAL_SELECTIVE) {
            SSM_LAUNCH(launch_fill_copy_f32(g->gA, nullptr, dn, st), "zero gA");
            SSM_LAUNCH(launch_fill_copy_f32(g->gdelta_bias, nullptr, (size_t)p.D, st), "zero gdelta_bias");
            SSM_LAUNCH(launch_zero_bytes(g->gBm, btn * p.esz, st), "zero gBm");
            SSM_LAUNCH(launch_zero_bytes(g->gC, btn * p.esz, st), "zero gC");
        } else if (p.mode == SSM_REAL_DENSE) {
            SSM_LAUNCH(launch_zero_bytes(g->gC, btn * 4, st), "zero gC");
        } else {
            if (p.mode == SSM_COMPLEX_SHARED) {
                SSM_LAUNCH(launch_fill_copy_f32(g->glam, nullptr, dn, st), "zero glam");
                SSM_LAUNCH(launch_fill_copy_f32(g->gtheta, nullptr, dn, st), "zero gtheta");
            }
            SSM_LAUNCH(launch_fill_copy_f32(g->gc, nullptr, 2 * dn, st), "zero gc");
        }
        return ok();
    }
    Carve cv(nullptr);
    if (p.mode == SSM_HEAD_SCALAR) {
        // the adjoint of the matrix form: chunk sums of the adjoint (the state pass on gy and C),
        // their reverse chain, then one workgroup per (chunk, head, batch); gB, gC and gA add
        // per-head terms in head order
        struct L2 {
            float* ckpt = nullptr;
            HeadFwdLayout fwd;
            float *gstate = nullptr, *decay = nullptr, *partB = nullptr, *partC = nullptr, *partA = nullptr;
        };
        const size_t hbnl = (size_t)p.H * p.B * p.N * p.L;
        auto layout = [&](Carve& c, bool have, bool wB, bool wC, bool wA, L2* l) {
            if (!have) {
                l->ckpt = c.take<float>((size_t)p.B * p.D * p.nchunks * p.N);
                head_fwd_layout(p, c, &l->fwd);
            }
            l->gstate = c.take<float>((size_t)p.B * p.D * p.nchunks * p.N);
            l->decay = c.take<float>((size_t)p.B * p.H * p.nchunks);
            if (wB) l->partB = c.take<float>(hbnl);
            if (wC) l->partC = c.take<float>(hbnl);
            if (wA) l->partA = c.take<float>((size_t)p.H * p.B * p.nchunks);
        };
        L2 sizing;
        layout(cv, false, true, true, true, &sizing);
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        L2 l;
        layout(real, in->ckpt != nullptr, g->gBm != nullptr, g->gC != nullptr, g->gA != nullptr, &l);
        const float* ckpt = in->ckpt;
        if (!ckpt) {
            if ((rc = run_head_fwd(a, p, l.fwd, nullptr, nullptr, l.ckpt, st))) return rc;
            ckpt = l.ckpt;
        }
        const int64_t e16 = 16 / (int64_t)p.esz;
        auto al = [](const void* ptr, int64_t bytes) { return ((uintptr_t)ptr % (uintptr_t)bytes) == 0; };
        // Q_c = C^T diag(e^s) dY for every chunk: the state pass with x = gy, B = C, weights e^(s_u)
        HeadParams hs{};
        hs.delta = a->delta; hs.x = in->gy; hs.A = a->A; hs.Bm = a->C; hs.C = a->C;
        copy_strides(hs.sdelta, p, SSM_V_DELTA); copy_strides(hs.sx, p, SSM_V_GY);
        copy_strides(hs.sBm, p, SSM_V_C); copy_strides(hs.sC, p, SSM_V_C);
        hs.sA = p.v.s[SSM_V_A][0];
        hs.state = l.gstate; hs.decay = l.decay;
        hs.B = (int)p.B; hs.H = (int)p.H; hs.P = (int)p.P; hs.L = (int)p.L; hs.N = (int)p.N; hs.nchunks = p.nchunks;
        hs.vx = al(in->gy, 16) && hs.sx[0] % e16 == 0 && hs.sx[1] % e16 == 0;
        hs.vb = al(a->C, 16) && hs.sBm[0] % e16 == 0 && hs.sBm[2] % e16 == 0;
        hs.bstate = 1;
        HeadBwdParams q{};
        q.delta = a->delta; q.x = a->x; q.A = a->A; q.Bm = a->Bm; q.C = a->C; q.gy = in->gy;
        q.ckpt = ckpt; q.gh_last = in->gh_last;
        copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sx, p, SSM_V_X); copy_strides(q.sgy, p, SSM_V_GY);
        copy_strides(q.sgx, p, SSM_V_GX); copy_strides(q.sgdelta, p, SSM_V_GDELTA);
        copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
        q.sA = p.v.s[SSM_V_A][0];
        q.gstate = l.gstate; q.decay = l.decay;
        q.gx = g->gx; q.gdelta = g->gdelta; q.gh0 = g->gh0;
        q.partB = l.partB; q.partC = l.partC; q.partA = l.partA;
        q.B = (int)p.B; q.H = (int)p.H; q.P = (int)p.P; q.L = (int)p.L; q.N = (int)p.N; q.nchunks = p.nchunks;
        q.vx = al(a->x, 16) && q.sx[0] % e16 == 0 && q.sx[1] % e16 == 0;
        q.vgy = hs.vx;
        q.vb = al(a->Bm, 16) && q.sBm[0] % e16 == 0 && q.sBm[2] % e16 == 0;
        q.vc = hs.vb;
        q.vgx = g->gx && al(g->gx, 4 * (int64_t)p.esz) && q.sgx[0] % 4 == 0 && q.sgx[1] % 4 == 0;
        SSM_LAUNCH(launch_head_state(hs, p.dtype, st), "head backward chunk sums (matrix cores)");
        SSM_LAUNCH(launch_head_rchain(q, st), "head backward chain over the chunks");
        SSM_LAUNCH(launch_head_bwd(q, p.dtype, st), "head backward (matrix cores)");
        if (g->gBm || g->gC)
            SSM_LAUNCH(launch_reduce_parts_btn(l.partB, l.partC, (int)p.H, (int)p.B, (int)p.N, (int)p.L, g->gBm,
                                               g->gC, p.dtype, st),
                       "gB gC: sums over the heads");
        if (g->gA)
            SSM_LAUNCH(launch_head_sum_rows(l.partA, g->gA, (int)p.H, (int)(p.B * p.nchunks), st),
                       "gA: sums over batch rows and chunks");
        return ok();
    }
    if (p.mode == SSM_REAL_SELECTIVE) {
        // workspace is sized for the worst case (checkpoints recomputed, every gradient wanted);
        // per-channel Bm, C have per-channel gradients: no channel-block partials
        SelBwdLayout sizing;
        sel_bwd_layout(p, false, !p.perd, !p.perd, true, true, cv, &sizing);
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        SelBwdLayout lay;  // only the buffers this call needs are non-null
        sel_bwd_layout(p, have_ckpt, g->gBm != nullptr && !p.perd, g->gC != nullptr && !p.perd, g->gA != nullptr,
                       g->gdelta_bias != nullptr, real, &lay);
        const float* ckpt = in->ckpt;
        if (!have_ckpt) {
            if ((rc = run_sel_fwd(a, p, lay.fwd, nullptr, nullptr, lay.ckpt, nullptr, st))) return rc;
            ckpt = lay.ckpt;
        }
        SelBwdParams q{};
        q.delta = a->delta; q.x = a->x; q.A = a->A; q.Bm = a->Bm; q.C = a->C;
        q.gy = in->gy; q.gh_last = in->gh_last; q.ckpt = ckpt; q.nu_in = lay.nu;
        q.gdelta = g->gdelta; q.gx = g->gx; q.gh0 = g->gh0;
        q.partB = lay.partB; q.partC = lay.partC; q.partA = lay.partA;
        q.segQ = lay.segQ; q.segR = lay.segR;
        q.B = (int)p.B; q.D = (int)p.D; q.L = (int)p.L; q.N = (int)p.N;
        q.ntiles = p.nchunks; q.tiles_per_seg = lay.tps; q.G = lay.G;
        q.vec = sel_vec(p, {a->delta, a->x, in->gy, g->gdelta, g->gx},
                        {SSM_V_DELTA, SSM_V_X, SSM_V_GY, SSM_V_GDELTA, SSM_V_GX});
        q.stepf = StepXform{a->delta_bias, a->delta_softplus};
        q.partBias = lay.partBias;
        copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sx, p, SSM_V_X); copy_strides(q.sgy, p, SSM_V_GY);
        copy_strides(q.sgx, p, SSM_V_GX); copy_strides(q.sgdelta, p, SSM_V_GDELTA);
        copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
        q.sA = p.v.s[SSM_V_A][0];
        q.bc_vec = sel_bc_vec(p, a->Bm, a->C);
        q.var = sel_var(p);
        if (p.perd) { q.gBm_pd = g->gBm; q.gC_pd = g->gC; }
        if (lay.G > 1) {
            SSM_LAUNCH(launch_sel_bwd(q, p.dtype, p.kpl, true, st), "selective backward summary");
            SSM_LAUNCH(launch_seg_combine_rev(lay.segQ, lay.segR, in->gh_last, lay.nu, (int)(p.B * p.D), lay.G,
                                              (int)p.N, st), "segment combine (reverse)");
        }
        SSM_LAUNCH(launch_sel_bwd(q, p.dtype, p.kpl, false, st), "selective backward");
        const int nblk = (int)cdiv(p.D, sel_bwd_rows());
        if ((g->gBm || g->gC) && !p.perd)
            SSM_LAUNCH(launch_reduce_parts_btn(g->gBm ? lay.partB : nullptr, g->gC ? lay.partC : nullptr, nblk,
                                               (int)p.B, (int)p.N, (int)p.L, g->gBm, g->gC, p.dtype, st),
                       "reduce gB gC");
        if (g->gA)
            SSM_LAUNCH(launch_reduce_parts_dn(lay.partA, (int)p.B, lay.G, (int)p.D, (int)p.N, g->gA, st),
                       "reduce gA");
        if (g->gdelta_bias)
            SSM_LAUNCH(launch_reduce_parts_dn(lay.partBias, (int)p.B, lay.G, (int)p.D, 1, g->gdelta_bias, st),
                       "reduce gdelta_bias");
        return ok();
    }
    if (p.mode == SSM_REAL_DENSE) {
        if ((rc = dense_bwd(a, p, in, g, cv, true, st))) return rc;
        if (need_only) { *need_only = cv.off; return ok(); }
        if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
        Carve real(ws);
        if ((rc = dense_bwd(a, p, in, g, real, false, st))) return rc;
        return ok();
    }
    if ((rc = cplx_bwd(a, p, in, g, cv, true, st))) return rc;
    if (need_only) { *need_only = cv.off; return ok(); }
    if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
    Carve real(ws);
    if ((rc = cplx_bwd(a, p, in, g, real, false, st))) return rc;
    return ok();
}

// ---------------------------------------------------------------------------
// ssm_impulse_sensitivity
// ---------------------------------------------------------------------------
// with_delta: also s_delta = d y[t_out] / d delta (ssm_output_sensitivity), which
// needs the forward checkpoints; s may then be NULL.
int impulse_impl(const ssm_scan_args* a, int64_t t_out, void* y, void* s, void* s_delta, bool with_delta,
                 void* ws, size_t ws_bytes, hipStream_t st, size_t* need_only) {
    ScanPlan p;
    int rc = validate_scan_args(a, &p, 256, E_SENS);
    if (rc) return rc;
    const char* name = with_delta ? "ssm_output_sensitivity" : "ssm_impulse_sensitivity";
    if (p.mode != SSM_REAL_SELECTIVE) return fail(SSM_ERR_UNSUPPORTED, "%s supports SSM_REAL_SELECTIVE only", name);
    if (t_out == -1) t_out = p.L - 1;
    if (t_out < 0 || t_out >= p.L) return fail(SSM_ERR_SHAPE, "t_out %lld outside [0, L)", (long long)t_out);
    if (p.empty) {   // no batch rows or channels: every output has zero elements
        if (need_only) *need_only = 0;
        return ok();
    }
    if (!need_only) {
        if (!with_delta && !s) return fail(SSM_ERR_NULL, "s is NULL");
        if (with_delta && !s_delta) return fail(SSM_ERR_NULL, "s_delta is NULL");
        const size_t BDL = p.B * p.D * p.L;
        if ((rc = check_align(s, p.esz, "s")) || (rc = check_align(y, p.esz, "y")) ||
            (rc = check_align(s_delta, p.esz, "s_delta")))
            return rc;
        if ((rc = check_overlaps(scan_inputs(a, p), {{y, BDL * p.esz, "y"}, {s, BDL * p.esz, "s"},
                                                     {s_delta, BDL * p.esz, "s_delta"}})))
            return rc;
    }
    // The forward's main pass forms the sensitivities itself when it runs anyway (y wanted, or the delta
    // sensitivity, which needs the states), the sequence is cut into segments (their summary pass gives the
    // tile sums first), N = 16 and the input term is Euler with shared B_t, C_t.
    const bool fusable = (with_delta || (y && s)) && p.N == 16 && sel_var(p) == kVarEuler;
    auto layout = [&](Carve& cv, SelFwdLayout* lay, float** tsum, double** send, float** ckpt) {
        sel_fwd_layout(p, cv, lay);
        *tsum = cv.take<float>((size_t)p.B * p.D * p.nchunks);
        *send = cv.take<double>((size_t)p.B * p.D * p.nchunks);
        const bool fused = fusable && lay->G > 1;
        *ckpt = with_delta && !fused ? cv.take<float>((size_t)p.B * p.D * p.nchunks * p.N) : nullptr;
    };
    Carve cv(nullptr);
    SelFwdLayout lay;
    float* tsum;
    double* send;
    float* ckpt;
    layout(cv, &lay, &tsum, &send, &ckpt);
    if (need_only) { *need_only = cv.off; return ok(); }
    if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
    Carve real(ws);
    layout(real, &lay, &tsum, &send, &ckpt);
    if (fusable && lay.G > 1) {
        // one pass forms y and the sensitivities: no checkpoints, no separate sensitivity kernel
        const FwdSens fs{s, with_delta ? s_delta : nullptr, send, (int)t_out};
        return run_sel_fwd(a, p, lay, y, nullptr, nullptr, tsum, st, &fs);
    }
    if (y || with_delta) {
        if ((rc = run_sel_fwd(a, p, lay, y, nullptr, ckpt, tsum, st))) return rc;
    } else {
        SSM_LAUNCH(launch_tile_dsum(a->delta, p.v.s[SSM_V_DELTA][0], p.v.s[SSM_V_DELTA][1],
                                    StepXform{a->delta_bias, a->delta_softplus}, tsum, (int)p.B, (int)p.D, (int)p.L,
                                    p.nchunks, p.kpl, p.dtype, st),
                   "tile sums");
    }
    SSM_LAUNCH(launch_sens_suffix(a->delta, p.v.s[SSM_V_DELTA][0], p.v.s[SSM_V_DELTA][1],
                                  StepXform{a->delta_bias, a->delta_softplus}, tsum, send, (int)p.B, (int)p.D, (int)p.L,
                                  p.nchunks, p.T, (int)t_out, p.dtype, st),
               "suffix sums");
    SensParams q{};
    q.delta = a->delta; q.A = a->A; q.Bm = a->Bm; q.C = a->C; q.send = send; q.s = s;
    q.x = a->x; q.ckpt = ckpt; q.s_delta = with_delta ? s_delta : nullptr;
    q.stepf = StepXform{a->delta_bias, a->delta_softplus};
    q.B = (int)p.B; q.D = (int)p.D; q.L = (int)p.L; q.N = (int)p.N; q.ntiles = p.nchunks; q.t_out = (int)t_out;
    q.vec = sel_vec(p, {a->delta, s, a->x, s_delta});
    copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sx, p, SSM_V_X);
    copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
    q.sA = p.v.s[SSM_V_A][0];
    SSM_LAUNCH(launch_sens(q, p.dtype, p.kpl, st), "sensitivity");
    return ok();
}

// ---------------------------------------------------------------------------
// ssm_sensitivity_rows
// ---------------------------------------------------------------------------
int sens_rows_impl(const ssm_scan_args* a, int64_t t0, int32_t rows, void* s, void* ws, size_t ws_bytes,
                   hipStream_t st, size_t* need_only) {
    ScanPlan p;
    int rc = validate_scan_args(a, &p, 64, E_SENS);
    if (rc) return rc;
    if (p.mode != SSM_REAL_SELECTIVE)
        return fail(SSM_ERR_UNSUPPORTED, "ssm_sensitivity_rows supports SSM_REAL_SELECTIVE only");
    if (p.T != 64) return fail(SSM_ERR_UNSUPPORTED, "ssm_sensitivity_rows runs 64-step tiles (chunk_len 0 or 64)");
    const int R = need_only ? kSensRowsMax : rows;
    if (!need_only) {
        if (R < 1 || R > kSensRowsMax)
            return fail(SSM_ERR_SHAPE, "rows %d outside [1, %d]", (int)R, kSensRowsMax);
        if (t0 < 0 || t0 + R > p.L)
            return fail(SSM_ERR_SHAPE, "output rows [%lld, %lld) outside [0, L=%lld)", (long long)t0,
                        (long long)(t0 + R), (long long)p.L);
    }
    if (p.empty) {   // no batch rows, channels or steps: s has zero elements
        if (need_only) *need_only = 0;
        return ok();
    }
    if (!need_only) {
        if (!s) return fail(SSM_ERR_NULL, "s is NULL");
        if ((rc = check_align(s, p.esz, "s"))) return rc;
        const size_t sb = (size_t)R * p.B * p.D * p.L * p.esz;
        if ((rc = check_overlaps(scan_inputs(a, p), {{s, sb, "s"}}))) return rc;
    }
    const size_t BD = (size_t)p.B * p.D;
    auto layout = [&](Carve& cv, float** tsum, double** send, float** w) {
        *tsum = cv.take<float>(BD * p.nchunks);
        *send = cv.take<double>(BD * p.nchunks);
        *w = cv.take<float>(BD * kSensRowsMax * p.N);
    };
    Carve cv(nullptr);
    float *tsum, *w;
    double* send;
    layout(cv, &tsum, &send, &w);
    if (need_only) { *need_only = cv.off; return ok(); }
    if ((rc = check_ws(ws, ws_bytes, cv.off))) return rc;
    Carve real(ws);
    layout(real, &tsum, &send, &w);
    const StepXform sx{a->delta_bias, a->delta_softplus};
    const int64_t sdb = p.v.s[SSM_V_DELTA][0], sdd = p.v.s[SSM_V_DELTA][1];
    SSM_LAUNCH(launch_tile_dsum(a->delta, sdb, sdd, sx, tsum, (int)p.B, (int)p.D, (int)p.L, p.nchunks, p.kpl, p.dtype,
                                st),
               "tile sums");
    SSM_LAUNCH(launch_sens_suffix(a->delta, sdb, sdd, sx, tsum, send, (int)p.B, (int)p.D, (int)p.L, p.nchunks, p.T,
                                  (int)t0, p.dtype, st),
               "suffix sums");
    SensRowsParams q{};
    q.delta = a->delta; q.A = a->A; q.Bm = a->Bm; q.C = a->C; q.send = send; q.w = w; q.s = s; q.stepf = sx;
    q.B = (int)p.B; q.D = (int)p.D; q.L = (int)p.L; q.N = (int)p.N; q.ntiles = p.nchunks; q.t0 = (int)t0; q.R = R;
    q.vec = sel_vec(p, {s});
    copy_strides(q.sdelta, p, SSM_V_DELTA); copy_strides(q.sBm, p, SSM_V_BM); copy_strides(q.sC, p, SSM_V_C);
    q.sA = p.v.s[SSM_V_A][0];
    q.bc_vec = sel_bc_vec(p, a->Bm, a->C);
    SSM_LAUNCH(launch_sens_rows_edge(q, false, p.dtype, st), "sensitivity rows (weights)");
    SSM_LAUNCH(launch_sens_rows(q, p.dtype, st), "sensitivity rows");
    SSM_LAUNCH(launch_sens_rows_edge(q, true, p.dtype, st), "sensitivity rows (tail)");
    return ok();
}

}  // namespace

#include "api_modes.inc"

// ===========================================================================
// allocation-free forward (ssm_scan_fwd_noalloc): the scratch memory the
// forward passes need (segment summaries and carries) lives in a static device
// array instead of a caller workspace.  Each device holds its own copy at its
// own address, found once per device with hipGetSymbolAddress; the array's
// name is only a host-side stand-in and is never passed to a kernel.
// ===========================================================================
static_assert(SSM_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SSM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `st` (the current device
// for the NULL stream), looked up on the first call for that device.
int scratch_for_stream(hipStream_t st, void** out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(SSM_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorName(e));
    dev = cur;
    if (st) {
        e = hipStreamGetDevice(st, &dev);
        if (e != hipSuccess) return fail(SSM_ERR_DEVICE, "hipStreamGetDevice: %s", hipGetErrorName(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(SSM_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(SSM_ERR_DEVICE, "hipSetDevice(%d): %s", dev, hipGetErrorName(e));
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) hipSetDevice(cur);
        if (e != hipSuccess || !ptr)
            return fail(SSM_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorName(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SSM_OK;
}

}  // namespace

// ===========================================================================
// exported C ABI
// ===========================================================================
extern "C" {

int ssm_workspace_bytes(int op, const void* args, size_t* out_bytes) {
    if (!out_bytes) return fail(SSM_ERR_NULL, "out_bytes is NULL");
    *out_bytes = 0;
    switch (op) {
        case SSM_OP_SCAN_FWD: return scan_fwd_impl((const ssm_scan_args*)args, nullptr, nullptr, 0, nullptr, out_bytes);
        case SSM_OP_SCAN_BWD: return scan_bwd_impl((const ssm_scan_args*)args, nullptr, nullptr, nullptr, 0, nullptr, out_bytes);
        case SSM_OP_IMPULSE:
            return impulse_impl((const ssm_scan_args*)args, -1, nullptr, nullptr, nullptr, false, nullptr, 0, nullptr,
                                out_bytes);
        case SSM_OP_OUTPUT_SENS:
            return impulse_impl((const ssm_scan_args*)args, -1, nullptr, nullptr, nullptr, true, nullptr, 0, nullptr,
                                out_bytes);
        case SSM_OP_PD_FWD: return pd_fwd_impl((const pd_scan_args*)args, nullptr, nullptr, 0, nullptr, out_bytes);
        case SSM_OP_PD_BWD: return pd_bwd_impl((const pd_scan_args*)args, nullptr, nullptr, nullptr, 0, nullptr, out_bytes);
        case SSM_OP_SENS_ROWS:
            return sens_rows_impl((const ssm_scan_args*)args, 0, 0, nullptr, nullptr, 0, nullptr, out_bytes);
        case SSM_OP_COMPLEX_RTRL:
            return rtrl_impl((const ssm_scan_args*)args, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, out_bytes);
        default: return fail(SSM_ERR_UNSUPPORTED, "unknown op %d", op);
    }
}

int ssm_scan_fwd(const ssm_scan_args* args, const ssm_scan_fwd_out* out, void* ws, size_t ws_bytes, void* stream) {
    return scan_fwd_impl(args, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int ssm_scan_fwd_noalloc(const ssm_scan_args* args, const ssm_scan_fwd_out* out, void* stream) {
    size_t need = 0;
    int rc = scan_fwd_impl(args, nullptr, nullptr, 0, nullptr, &need);   // host-only: validation and sizing
    if (rc) return rc;
    if (need > (size_t)SSM_NOALLOC_SCRATCH_BYTES)
        return fail(SSM_ERR_WORKSPACE, "the forward needs %zu bytes of scratch; the static scratch holds %zu",
                    need, (size_t)SSM_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((rc = scratch_for_stream((hipStream_t)stream, &ws))) return rc;
    // no part of the scratch has to start at zero: every pass writes what it later reads
    return scan_fwd_impl(args, out, ws, SSM_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream, nullptr);
}
int ssm_scan_bwd(const ssm_scan_args* args, const ssm_scan_bwd_in* in, const ssm_scan_grads* grads, void* ws,
                 size_t ws_bytes, void* stream) {
    return scan_bwd_impl(args, in, grads, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int ssm_impulse_sensitivity(const ssm_scan_args* args, int64_t t_out, void* y, void* s, void* ws, size_t ws_bytes,
                            void* stream) {
    return impulse_impl(args, t_out, y, s, nullptr, false, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int ssm_output_sensitivity(const ssm_scan_args* args, int64_t t_out, void* y, void* s_x, void* s_delta, void* ws,
                           size_t ws_bytes, void* stream) {
    return impulse_impl(args, t_out, y, s_x, s_delta, true, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int ssm_sensitivity_rows(const ssm_scan_args* args, int64_t t_out0, int32_t rows, void* s, void* ws,
                         size_t ws_bytes, void* stream) {
    return sens_rows_impl(args, t_out0, rows, s, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int ssm_complex_rtrl(const ssm_scan_args* args, const void* gy, const float* gh_last, void* y, float* glam,
                     float* gtheta, void* ws, size_t ws_bytes, void* stream) {
    return rtrl_impl(args, gy, gh_last, y, glam, gtheta, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int pd_scan_fwd(const pd_scan_args* args, const pd_scan_fwd_out* out, void* ws, size_t ws_bytes, void* stream) {
    return pd_fwd_impl(args, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}
int pd_scan_bwd(const pd_scan_args* args, const pd_scan_bwd_in* in, const pd_scan_grads* grads, void* ws,
                size_t ws_bytes, void* stream) {
    return pd_bwd_impl(args, in, grads, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

int ssm_profile_begin(int max_launches) {
    if (max_launches < 0) return fail(SSM_ERR_SHAPE, "max_launches < 0");
    Profile& p = g_prof;
    while ((int)p.ev.size() < 2 * max_launches) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return fail(SSM_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorName(err));
        p.ev.push_back(e);
    }
    p.names.assign(max_launches, nullptr);
    p.cap = max_launches;
    p.n = 0;
    p.on = max_launches > 0;
    return ok();
}
int ssm_profile_end(int* n_launches, float* ms, const char** names, int capacity) {
    Profile& p = g_prof;
    p.on = false;
    if (n_launches) *n_launches = p.n;
    if (p.n > 0) {
        hipError_t err = hipEventSynchronize(p.ev[2 * p.n - 1]);
        if (err != hipSuccess) return fail(SSM_ERR_DEVICE, "hipEventSynchronize: %s", hipGetErrorName(err));
    }
    for (int i = 0; i < p.n && i < capacity; ++i) {
        float t = 0.0f;
        hipError_t err = hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]);
        if (err != hipSuccess) return fail(SSM_ERR_DEVICE, "hipEventElapsedTime: %s", hipGetErrorName(err));
        if (ms) ms[i] = t;
        if (names) names[i] = p.names[i];
    }
    return ok();
}

int ssm_roof_probe(int kind, int chains, int waves, int iters, float* sink, double* lane_ops_per_s, void* stream) {
    if (!sink || !lane_ops_per_s) return fail(SSM_ERR_NULL, "sink and lane_ops_per_s are required");
    if (kind < 0 || kind > 7) return fail(SSM_ERR_UNSUPPORTED, "unknown probe kind %d", kind);
    if (chains != 4 && chains != 8) return fail(SSM_ERR_UNSUPPORTED, "chains must be 4 or 8");
    if (kind == 3 && chains != 4) return fail(SSM_ERR_UNSUPPORTED, "the DPP probe runs 4 chains");
    if (kind == 7 && chains != 8) return fail(SSM_ERR_UNSUPPORTED, "the v_fmac_f32 probe runs 8 chains");
    if (waves < 1 || waves > 65536 || iters < 1 || iters > (1 << 24))
        return fail(SSM_ERR_SHAPE, "waves in [1, 65536] and iters in [1, 2^24] required");
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t e0, e1;
    hipError_t e = hipEventCreate(&e0);
    if (e != hipSuccess) return fail(SSM_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorName(e));
    if ((e = hipEventCreate(&e1)) != hipSuccess) {
        hipEventDestroy(e0);
        return fail(SSM_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorName(e));
    }
    float ms = 0.0f;
    if ((e = hipEventRecord(e0, st)) == hipSuccess && (e = launch_roof(kind, chains, waves, iters, sink, st)) == hipSuccess &&
        (e = hipEventRecord(e1, st)) == hipSuccess && (e = hipEventSynchronize(e1)) == hipSuccess)
        e = hipEventElapsedTime(&ms, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    if (e != hipSuccess) return fail(SSM_ERR_DEVICE, "roof probe: %s", hipGetErrorName(e));
    *lane_ops_per_s = (double)waves * 64.0 * roof_instrs_per_lane(kind, chains, iters) / (ms * 1e-3);
    return ok();
}

const char* ssm_status_string(int status) {
    switch (status) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_NULL: return "SSM_ERR_NULL";
        case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE";
        case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE";
        case SSM_ERR_LAYOUT: return "SSM_ERR_LAYOUT";
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
        case SSM_ERR_DEVICE: return "SSM_ERR_DEVICE";
        default: return "SSM_ERR_UNKNOWN";
    }
}
const char* ssm_last_error_detail(void) { return g_detail.c_str(); }
int ssm_abi_version(void) { return SSM_ABI_VERSION; }

}  // extern "C"
