// qkv_epilogue.hip -- fused attention-input epilogue for MI355X (gfx950).
//
// One launch per layer does, for every token: bias add on q, k and v; NeoX
// rotary embedding on q and k; write-back of all three sections; and the K/V
// cache row store (f32, or f16 rounded to nearest even).  The operation is the
// one of page "73 · D3-8 — G4 FusedQKV ported to CUDA" (minfer CUDA
// optimization steps), §2 and §3.2 Excerpt A; the cache layout (one row of
// n_kv_head*head_dim elements per position) is that of page "07 · The
// allocator", §2.5.  The page's own kernel (one thread per rope pair or v
// element, cos/sin recomputed per pair) is prior art only; the mapping here is
// built for 64-lane CDNA4 wavefronts and HBM3E:
//
//  * Work unit.  A unit is two W-wide slots of one token's row.  For q and k a
//    unit is W rotary pairs of one head: elements [i0, i0+W) and
//    [i0+half, i0+half+W), so both halves of a pair arrive in the same lane
//    from two 16-byte loads and no cross-lane exchange is needed.  For v a
//    unit is 2W consecutive elements.  Units of a token are laid out q, k, v;
//    the launch walks the flat range [0, nt*units_per_token) so tokens and
//    sequences (prefill, batched decode) fill the chip the same way.
//  * Each thread owns UPT units strided by the workgroup size, so a wave's
//    loads cover whole 128-byte lines; every load of a thread is issued before
//    any arithmetic.
//  * cos/sin are computed once per (token, pair index) per workgroup, in double
//    precision, rounded to f32 and kept in LDS; the inverse frequencies ride in
//    the kernel arguments (computed on the host once per theta/head_dim).
//  * The rotation is evaluated in double: the products of two f32 values are
//    exact in double, so x0*c - x1*s is rounded once there and once to f32
//    whether or not the compiler fuses it into an FMA.
//  * f16 stores convert each element with the round-to-nearest-even conversion
//    and store W halves per instruction; the round-toward-zero pack
//    conversion is never used.
//  * A token whose position (or slot) is out of range gets its q/k/v written
//    back but no cache row; the kernel ORs a bit into a device error word
//    (page "07 · The allocator", §3.2 Excerpt 8: a position beyond the cache
//    is a hard error, never a silent overflow).
//
// Everything is launched asynchronously on the caller's stream; nothing here
// synchronizes except qkv_epilogue_status.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "qkv_epilogue.h"

namespace {

constexpr int kMaxHalf = QKV_MAX_HEAD_DIM / 2;
constexpr int kBlock = 256;

// Inverse-frequency table passed by value in the kernel arguments.
struct InvTable {
    float v[kMaxHalf];
};

struct KParams {
    float *x[3];          // q, k, v section bases
    const float *b[3];    // biases
    const int32_t *pos;
    const int32_t *slot;  // may be null
    void *cache[2];       // K, V (index sec-1)
    unsigned int *err;
    int64_t ld[3];
    int64_t n_ctx;
    int64_t n_slots;
    int64_t nkt;
    uint32_t total;       // nt * U
    int nt;
    int hd;
    int half;
    int uph;              // rope units per head = half / W
    int qu;               // q rope units per token
    int qku;              // q + k rope units per token
    int U;                // units per token
    int max_tok;          // tokens one workgroup may touch (LDS sizing)
};

template <int W>
struct alignas(4 * W) FVec {
    float e[W];
};

template <int W>
struct alignas(2 * W) HVec {
    _Float16 e[W];
};

template <int W>
__device__ __forceinline__ FVec<W> ld_vec(const float *p)
{
    return *reinterpret_cast<const FVec<W> *>(p);
}

template <int W>
__device__ __forceinline__ void st_vec(float *p, const FVec<W> &v)
{
    *reinterpret_cast<FVec<W> *>(p) = v;
}

template <int W, bool F16>
__device__ __forceinline__ void st_cache(void *cache, int64_t off, const FVec<W> &v)
{
    if constexpr (F16) {
        HVec<W> h;
#pragma unroll
        for (int e = 0; e < W; ++e)
            h.e[e] = static_cast<_Float16>(v.e[e]);  // v_cvt_f16_f32: RNE
        *reinterpret_cast<HVec<W> *>(static_cast<_Float16 *>(cache) + off) = h;
    } else {
        *reinterpret_cast<FVec<W> *>(static_cast<float *>(cache) + off) = v;
    }
}

// LDS layout: int64 row[max_tok] | float cos[max_tok*half] | float sin[...]
__host__ __device__ inline int lds_row_bytes(int max_tok)
{
    return ((max_tok * 8) + 15) & ~15;
}

template <int W, bool F16, int UPT>
__global__ __launch_bounds__(kBlock) void qkv_epilogue_kernel(KParams p, InvTable inv)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    int64_t *s_row = reinterpret_cast<int64_t *>(lds_raw);
    float *s_cos = reinterpret_cast<float *>(lds_raw + lds_row_bytes(p.max_tok));
    float *s_sin = s_cos + p.max_tok * p.half;

    const uint32_t tid = threadIdx.x;
    const uint32_t g0 = blockIdx.x * (uint32_t)(kBlock * UPT);
    const uint32_t g_last = min(g0 + (uint32_t)(kBlock * UPT), p.total) - 1u;
    const int t_lo = (int)(g0 / (uint32_t)p.U);
    const int ntok = (int)(g_last / (uint32_t)p.U) - t_lo + 1;

    // ---- phase 1: decode this thread's units and issue every load ---------
    int sec[UPT];        // 0 q, 1 k, 2 v, -1 none
    int tl[UPT];         // token index local to the workgroup
    int col[UPT];        // column of the first slot inside the section row
    int i0[UPT];         // first pair index (rope units)
    FVec<W> xa[UPT], xb[UPT], ba[UPT], bb[UPT];

#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const uint32_t g = g0 + (uint32_t)u * kBlock + tid;
        sec[u] = -1;
        if (g < p.total) {
            const int t = (int)(g / (uint32_t)p.U);
            int r = (int)(g - (uint32_t)t * (uint32_t)p.U);
            int s, c, i, d1;
            if (r < p.qku) {
                s = r < p.qu ? 0 : 1;
                if (s) r -= p.qu;
                const int h = r / p.uph;
                i = (r - h * p.uph) * W;
                c = h * p.hd + i;
                d1 = p.half;
            } else {
                s = 2;
                i = 0;
                c = (r - p.qku) * (2 * W);
                d1 = W;
            }
            sec[u] = s;
            tl[u] = t - t_lo;
            col[u] = c;
            i0[u] = i;
            const float *xp = p.x[s] + (int64_t)t * p.ld[s] + c;
            const float *bp = p.b[s] + c;
            xa[u] = ld_vec<W>(xp);
            xb[u] = ld_vec<W>(xp + d1);
            ba[u] = ld_vec<W>(bp);
            bb[u] = ld_vec<W>(bp + d1);
        }
    }

    // ---- phase 2: per (token, pair) cos/sin and per-token cache rows -------
    const int ent = ntok * p.half;
    for (int e = (int)tid; e < ent; e += kBlock) {
        const int tk = e / p.half;
        const int i = e - tk * p.half;
        const float a = (float)p.pos[t_lo + tk] * inv.v[i];   // f32 angle
        double sd, cd;
        sincos((double)a, &sd, &cd);
        s_cos[e] = (float)cd;
        s_sin[e] = (float)sd;
    }
    for (int e = (int)tid; e < ntok; e += kBlock) {
        const int t = t_lo + e;
        const int64_t ps = p.pos[t];
        const int64_t sl = p.slot ? (int64_t)p.slot[t] : 0;
        int64_t row = -1;
        if (ps >= 0 && ps < p.n_ctx && sl >= 0 && sl < p.n_slots)
            row = sl * p.n_ctx + ps;
        else
            atomicOr(p.err, 1u);
        s_row[e] = row;
    }
    __syncthreads();

    // ---- phase 3: bias, rotate, write back, store cache rows ---------------
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const int s = sec[u];
        if (s < 0)
            continue;
        const int t = t_lo + tl[u];
        FVec<W> ra, rb;
#pragma unroll
        for (int e = 0; e < W; ++e) {
            ra.e[e] = xa[u].e[e] + ba[u].e[e];
            rb.e[e] = xb[u].e[e] + bb[u].e[e];
        }
        int d1 = W;
        if (s < 2) {
            d1 = p.half;
            const int ci = tl[u] * p.half + i0[u];
            const FVec<W> cs = ld_vec<W>(s_cos + ci);
            const FVec<W> sn = ld_vec<W>(s_sin + ci);
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const double x0 = (double)ra.e[e];
                const double x1 = (double)rb.e[e];
                const double c = (double)cs.e[e];
                const double sv = (double)sn.e[e];
                ra.e[e] = (float)(x0 * c - x1 * sv);
                rb.e[e] = (float)(x0 * sv + x1 * c);
            }
        }
        float *xp = p.x[s] + (int64_t)t * p.ld[s] + col[u];
        st_vec<W>(xp, ra);
        st_vec<W>(xp + d1, rb);
        if (s > 0) {
            const int64_t row = s_row[tl[u]];
            if (row >= 0) {
                const int64_t off = row * p.nkt + col[u];
                st_cache<W, F16>(p.cache[s - 1], off, ra);
                st_cache<W, F16>(p.cache[s - 1], off + d1, rb);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Plan {
    int W;
    int U;
    int UPT;
    int64_t grid;
    int lds;
    int max_tok;
    int half;
    int64_t nqt, nkt;
    int64_t ld[3];
    int64_t n_ctx, n_slots;
};

void set_msg(char *msg, size_t len, const char *fmt, ...)
{
    if (!msg || !len)
        return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, len, fmt, ap);
    va_end(ap);
}

struct Span {
    uintptr_t base;  // byte address of the first element
    int64_t ld;      // row stride in bytes (0 for a contiguous block)
    int64_t width;   // bytes per row
    int64_t rows;
    const char *name;
};

int64_t floor_div(int64_t a, int64_t b)  // b > 0
{
    int64_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// Do two (possibly strided) row sets share a byte?  Row i of a covers
// [a.base + i*ld, a.base + i*ld + width).  Exact for equal strides (a single
// row takes the other set's stride); conservative (hull test) otherwise.
bool spans_overlap(Span a, Span b)
{
    if (a.rows <= 0 || b.rows <= 0 || a.width <= 0 || b.width <= 0)
        return false;
    const uintptr_t a_end = a.base + (uintptr_t)((a.rows - 1) * a.ld + a.width);
    const uintptr_t b_end = b.base + (uintptr_t)((b.rows - 1) * b.ld + b.width);
    if (a_end <= b.base || b_end <= a.base)
        return false;
    if (a.rows == 1)
        a.ld = b.ld;
    if (b.rows == 1)
        b.ld = a.ld;
    if (a.rows == 1 && b.rows == 1)
        return true;
    if (a.ld != b.ld || a.ld <= 0)
        return true;
    // Rows i of a and j of b meet iff -b.width < d + m*L < a.width, m = j - i,
    // d = b.base - a.base; d + m*L grows with m, so only the smallest m above
    // the lower bound can satisfy the upper one.
    const int64_t L = a.ld;
    const int64_t d = (int64_t)b.base - (int64_t)a.base;
    int64_t m = floor_div(-b.width - d, L) + 1;
    if (m < -(a.rows - 1))
        m = -(a.rows - 1);
    if (m > b.rows - 1)
        return false;
    return d + m * L < a.width;
}

int check_and_plan(const qkv_epilogue_args_t *a, int64_t n_ctx_default, Plan *pl, char *msg,
                   size_t mlen)
{
    if (!a) {
        set_msg(msg, mlen, "args is NULL");
        return QKV_ERR_INVALID_ARG;
    }
    if (a->rope_style != QKV_ROPE_NEOX) {
        set_msg(msg, mlen,
                "rope_style %d not supported: only NeoX pairing (i, i+head_dim/2) is "
                "implemented",
                a->rope_style);
        return QKV_ERR_UNSUPPORTED;
    }
    if (a->nt < 0) {
        set_msg(msg, mlen, "nt must be >= 0, got %d", a->nt);
        return QKV_ERR_INVALID_ARG;
    }
    if (a->n_head < 1 || a->n_kv_head < 1) {
        set_msg(msg, mlen, "n_head and n_kv_head must be >= 1, got %d and %d", a->n_head,
                a->n_kv_head);
        return QKV_ERR_INVALID_ARG;
    }
    if (a->head_dim <= 0 || (a->head_dim & 1) || a->head_dim > QKV_MAX_HEAD_DIM) {
        set_msg(msg, mlen, "head_dim must be even and in [2, %d], got %d", QKV_MAX_HEAD_DIM,
                a->head_dim);
        return QKV_ERR_INVALID_ARG;
    }
    if (!(a->theta > 0.0f) || !std::isfinite(a->theta)) {
        set_msg(msg, mlen, "theta must be finite and > 0, got %g", (double)a->theta);
        return QKV_ERR_INVALID_ARG;
    }
    if (a->cache_dtype != QKV_CACHE_F32 && a->cache_dtype != QKV_CACHE_F16) {
        set_msg(msg, mlen, "cache_dtype must be 0 (f32) or 1 (f16), got %d", a->cache_dtype);
        return QKV_ERR_INVALID_ARG;
    }
    const int64_t nqt = (int64_t)a->n_head * a->head_dim;
    const int64_t nkt = (int64_t)a->n_kv_head * a->head_dim;
    if (a->ld_q < 0 || a->ld_k < 0 || a->ld_v < 0) {
        set_msg(msg, mlen, "row strides must be >= 0");
        return QKV_ERR_INVALID_ARG;
    }
    const int64_t ldq = a->ld_q ? a->ld_q : nqt;
    const int64_t ldk = a->ld_k ? a->ld_k : nkt;
    const int64_t ldv = a->ld_v ? a->ld_v : nkt;
    if (ldq < nqt || ldk < nkt || ldv < nkt) {
        set_msg(msg, mlen, "row stride below row width (ld_q %lld < %lld, ld_k %lld / ld_v %lld < %lld)",
                (long long)ldq, (long long)nqt, (long long)ldk, (long long)ldv, (long long)nkt);
        return QKV_ERR_INVALID_ARG;
    }
    if (a->n_ctx < 0 || a->n_slots < 0) {
        set_msg(msg, mlen, "n_ctx and n_slots must be >= 0");
        return QKV_ERR_INVALID_ARG;
    }
    const int64_t n_ctx = a->n_ctx ? a->n_ctx : n_ctx_default;
    const int64_t n_slots = a->n_slots ? a->n_slots : 1;
    if (n_ctx < 1) {
        set_msg(msg, mlen, "n_ctx must be >= 1");
        return QKV_ERR_INVALID_ARG;
    }
    const int cb = a->cache_dtype == QKV_CACHE_F16 ? 2 : 4;
    if (n_slots > INT64_MAX / n_ctx || n_slots * n_ctx > INT64_MAX / (nkt * cb)) {
        set_msg(msg, mlen, "cache size n_slots*n_ctx*nkt overflows");
        return QKV_ERR_INVALID_ARG;
    }

    pl->half = a->head_dim / 2;
    pl->nqt = nqt;
    pl->nkt = nkt;
    pl->ld[0] = ldq;
    pl->ld[1] = ldk;
    pl->ld[2] = ldv;
    pl->n_ctx = n_ctx;
    pl->n_slots = n_slots;
    pl->W = 1;
    pl->U = 0;
    pl->UPT = 1;
    pl->grid = 0;
    pl->lds = 0;
    pl->max_tok = 0;

    if (a->nt == 0)
        return QKV_OK;

    struct {
        const void *p;
        const char *n;
    } ptrs[] = {{a->q, "q"},   {a->k, "k"},   {a->v, "v"},   {a->bq, "bq"},         {a->bk, "bk"},
                {a->bv, "bv"}, {a->pos, "pos"}, {a->kcache, "kcache"}, {a->vcache, "vcache"}};
    for (auto &e : ptrs) {
        if (!e.p) {
            set_msg(msg, mlen, "%s is NULL", e.n);
            return QKV_ERR_INVALID_ARG;
        }
    }
    for (const float *f : {(const float *)a->q, (const float *)a->k, (const float *)a->v, a->bq, a->bk, a->bv}) {
        if ((uintptr_t)f % 4) {
            set_msg(msg, mlen, "f32 tensor pointer not 4-byte aligned");
            return QKV_ERR_INVALID_ARG;
        }
    }
    if ((uintptr_t)a->pos % 4 || (a->slot && (uintptr_t)a->slot % 4)) {
        set_msg(msg, mlen, "pos/slot pointer not 4-byte aligned");
        return QKV_ERR_INVALID_ARG;
    }
    if ((uintptr_t)a->kcache % cb || (uintptr_t)a->vcache % cb) {
        set_msg(msg, mlen, "cache pointer not aligned to its %d-byte element", cb);
        return QKV_ERR_INVALID_ARG;
    }

    // overlap checks on byte ranges
    const int64_t nt = a->nt;
    const int64_t cache_bytes = n_slots * n_ctx * nkt * cb;
    Span outs[5] = {
        {(uintptr_t)a->q, ldq * 4, nqt * 4, nt, "q"},
        {(uintptr_t)a->k, ldk * 4, nkt * 4, nt, "k"},
        {(uintptr_t)a->v, ldv * 4, nkt * 4, nt, "v"},
        {(uintptr_t)a->kcache, 0, cache_bytes, 1, "kcache"},
        {(uintptr_t)a->vcache, 0, cache_bytes, 1, "vcache"},
    };
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (spans_overlap(outs[i], outs[j])) {
                set_msg(msg, mlen, "%s and %s overlap", outs[i].name, outs[j].name);
                return QKV_ERR_ALIAS;
            }
    Span ins[5] = {
        {(uintptr_t)a->bq, 0, nqt * 4, 1, "bq"},
        {(uintptr_t)a->bk, 0, nkt * 4, 1, "bk"},
        {(uintptr_t)a->bv, 0, nkt * 4, 1, "bv"},
        {(uintptr_t)a->pos, 0, nt * 4, 1, "pos"},
        {(uintptr_t)a->slot, 0, a->slot ? nt * 4 : 0, 1, "slot"},
    };
    for (auto &in : ins)
        for (auto &o : outs)
            if (spans_overlap(in, o)) {
                set_msg(msg, mlen, "read-only %s overlaps output %s", in.name, o.name);
                return QKV_ERR_ALIAS;
            }

    // kernel variant: 16-byte vectors when every slot is 16-byte aligned
    bool vec = (a->head_dim % 8) == 0;
    for (const float *f : {(const float *)a->q, (const float *)a->k, (const float *)a->v, a->bq, a->bk, a->bv})
        vec = vec && ((uintptr_t)f % 16) == 0;
    vec = vec && (ldq % 4) == 0 && (ldk % 4) == 0 && (ldv % 4) == 0;
    vec = vec && ((uintptr_t)a->kcache % (4 * cb)) == 0 && ((uintptr_t)a->vcache % (4 * cb)) == 0;
    const int W = vec ? 4 : 1;
    const int half = a->head_dim / 2;
    const int64_t U = (int64_t)(a->n_head + a->n_kv_head) * (half / W) + nkt / (2 * W);
    const int64_t total = U * nt;
    if (total > (int64_t)INT32_MAX - (int64_t)kBlock * 8) {
        set_msg(msg, mlen, "launch too large: %lld work units (split the tokens)", (long long)total);
        return QKV_ERR_INVALID_ARG;
    }
    // Units per thread: keep >= 1024 workgroups (4 per CU) when possible.
    int upt = 1;
    while (upt < 4 && total / ((int64_t)kBlock * upt * 2) >= 1024)
        upt *= 2;
    const int64_t span = (int64_t)kBlock * upt;
    int64_t max_tok = (span + U - 1) / U + 1;
    if (max_tok > nt)
        max_tok = nt;
    pl->W = W;
    pl->U = (int)U;
    pl->UPT = upt;
    pl->grid = (total + span - 1) / span;
    pl->max_tok = (int)max_tok;
    pl->lds = lds_row_bytes((int)max_tok) + (int)(2 * max_tok * half * 4);
    if (pl->lds > 64 * 1024) {
        set_msg(msg, mlen, "internal: LDS plan %d bytes too large", pl->lds);
        return QKV_ERR_INVALID_ARG;
    }
    return QKV_OK;
}

void host_inv_freq(float theta, int head_dim, float *out)
{
    const int half = head_dim / 2;
    for (int i = 0; i < half; ++i)
        out[i] = (float)std::pow((double)theta, -(double)(2 * i) / (double)head_dim);
}

template <int W, bool F16, int UPT>
hipError_t launch_t(const KParams &kp, const InvTable &inv, int64_t grid, int lds, hipStream_t st)
{
    hipLaunchKernelGGL((qkv_epilogue_kernel<W, F16, UPT>), dim3((unsigned)grid), dim3(kBlock),
                       (unsigned)lds, st, kp, inv);
    return hipGetLastError();
}

template <int W, bool F16>
hipError_t launch_w(const KParams &kp, const InvTable &inv, int upt, int64_t grid, int lds,
                    hipStream_t st)
{
    switch (upt) {
    case 1: return launch_t<W, F16, 1>(kp, inv, grid, lds, st);
    case 2: return launch_t<W, F16, 2>(kp, inv, grid, lds, st);
    default: return launch_t<W, F16, 4>(kp, inv, grid, lds, st);
    }
}

}  // namespace

struct qkv_epilogue {
    int device;
    int64_t n_ctx;
    hipStream_t stream;
    hipStream_t last_stream;
    unsigned int *d_err;
    float inv_theta;
    int inv_hd;
    InvTable inv;
    char msg[512];
};

namespace {

int fail(qkv_epilogue *h, int code, const char *fmt, ...)
{
    if (h) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(h->msg, sizeof h->msg, fmt, ap);
        va_end(ap);
    }
    return code;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t set(int dev)
    {
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess)
            return e;
        if (prev != dev) {
            changed = true;
            return hipSetDevice(dev);
        }
        return hipSuccess;
    }
    ~DeviceGuard()
    {
        if (changed)
            (void)hipSetDevice(prev);
    }
};

}  // namespace

extern "C" {

int qkv_epilogue_create(qkv_epilogue_t **out, const qkv_epilogue_config_t *cfg)
{
    if (!out)
        return QKV_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg || cfg->n_ctx < 1 || cfg->device < 0)
        return QKV_ERR_INVALID_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0)
        return QKV_ERR_HIP;
    if (cfg->device >= ndev)
        return QKV_ERR_INVALID_ARG;
    qkv_epilogue *h = new (std::nothrow) qkv_epilogue();
    if (!h)
        return QKV_ERR_HIP;
    h->device = cfg->device;
    h->n_ctx = cfg->n_ctx;
    h->stream = static_cast<hipStream_t>(cfg->stream);
    h->last_stream = h->stream;
    h->inv_theta = 0.0f;
    h->inv_hd = 0;
    h->msg[0] = 0;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&h->d_err), 16);
    if (e == hipSuccess)
        e = hipMemset(h->d_err, 0, 16);
    if (e != hipSuccess) {
        if (h->d_err)
            (void)hipFree(h->d_err);
        delete h;
        return QKV_ERR_HIP;
    }
    *out = h;
    return QKV_OK;
}

int qkv_epilogue_run_ex(qkv_epilogue_t *h, const qkv_epilogue_args_t *a)
{
    if (!h)
        return QKV_ERR_INVALID_ARG;
    h->msg[0] = 0;
    Plan pl;
    int rc = check_and_plan(a, h->n_ctx, &pl, h->msg, sizeof h->msg);
    if (rc != QKV_OK)
        return rc;
    if (a->nt == 0)
        return QKV_OK;

    if (h->inv_hd != a->head_dim || h->inv_theta != a->theta) {
        host_inv_freq(a->theta, a->head_dim, h->inv.v);
        h->inv_hd = a->head_dim;
        h->inv_theta = a->theta;
    }

    KParams kp;
    kp.x[0] = a->q;
    kp.x[1] = a->k;
    kp.x[2] = a->v;
    kp.b[0] = a->bq;
    kp.b[1] = a->bk;
    kp.b[2] = a->bv;
    kp.pos = a->pos;
    kp.slot = a->slot;
    kp.cache[0] = a->kcache;
    kp.cache[1] = a->vcache;
    kp.err = h->d_err;
    kp.ld[0] = pl.ld[0];
    kp.ld[1] = pl.ld[1];
    kp.ld[2] = pl.ld[2];
    kp.n_ctx = pl.n_ctx;
    kp.n_slots = pl.n_slots;
    kp.nkt = pl.nkt;
    kp.total = (uint32_t)((int64_t)pl.U * a->nt);
    kp.nt = a->nt;
    kp.hd = a->head_dim;
    kp.half = pl.half;
    kp.uph = pl.half / pl.W;
    kp.qu = a->n_head * kp.uph;
    kp.qku = (a->n_head + a->n_kv_head) * kp.uph;
    kp.U = pl.U;
    kp.max_tok = pl.max_tok;

    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    const bool f16 = a->cache_dtype == QKV_CACHE_F16;
    if (pl.W == 4)
        e = f16 ? launch_w<4, true>(kp, h->inv, pl.UPT, pl.grid, pl.lds, st)
                : launch_w<4, false>(kp, h->inv, pl.UPT, pl.grid, pl.lds, st);
    else
        e = f16 ? launch_w<1, true>(kp, h->inv, pl.UPT, pl.grid, pl.lds, st)
                : launch_w<1, false>(kp, h->inv, pl.UPT, pl.grid, pl.lds, st);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    h->last_stream = st;
    return QKV_OK;
}

int qkv_epilogue_run(qkv_epilogue_t *h, float *q, float *k, float *v, const float *bq,
                     const float *bk, const float *bv, const int32_t *pos, void *kcache,
                     void *vcache, int nt, int n_head, int n_kv_head, int head_dim, float theta,
                     int cache_dtype)
{
    qkv_epilogue_args_t a;
    std::memset(&a, 0, sizeof a);
    a.q = q;
    a.k = k;
    a.v = v;
    a.bq = bq;
    a.bk = bk;
    a.bv = bv;
    a.pos = pos;
    a.kcache = kcache;
    a.vcache = vcache;
    a.nt = nt;
    a.n_head = n_head;
    a.n_kv_head = n_kv_head;
    a.head_dim = head_dim;
    a.theta = theta;
    a.cache_dtype = cache_dtype;
    a.rope_style = QKV_ROPE_NEOX;
    return qkv_epilogue_run_ex(h, &a);
}

int qkv_epilogue_status(qkv_epilogue_t *h)
{
    if (!h)
        return QKV_ERR_INVALID_ARG;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    unsigned int word = 0;
    if (e == hipSuccess)
        e = hipStreamSynchronize(h->last_stream);
    if (e == hipSuccess)
        e = hipMemcpy(&word, h->d_err, sizeof word, hipMemcpyDeviceToHost);
    if (e == hipSuccess && word)
        e = hipMemset(h->d_err, 0, sizeof word);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "status: %s", hipGetErrorString(e));
    if (word & 1u)
        return fail(h, QKV_ERR_POSITION_RANGE,
                    "a token's position was outside [0, n_ctx) or its slot outside [0, n_slots); "
                    "its cache rows were not written");
    return QKV_OK;
}

const char *qkv_epilogue_last_error(const qkv_epilogue_t *h)
{
    return h ? h->msg : "NULL handle";
}

void qkv_epilogue_destroy(qkv_epilogue_t *h)
{
    if (!h)
        return;
    DeviceGuard g;
    if (g.set(h->device) == hipSuccess && h->d_err)
        (void)hipFree(h->d_err);
    delete h;
}

int qkv_epilogue_inv_freq(float theta, int head_dim, float *out)
{
    if (!out || head_dim <= 0 || (head_dim & 1) || head_dim > QKV_MAX_HEAD_DIM ||
        !(theta > 0.0f) || !std::isfinite(theta))
        return QKV_ERR_INVALID_ARG;
    host_inv_freq(theta, head_dim, out);
    return QKV_OK;
}

int qkv_epilogue_check_args(const qkv_epilogue_args_t *a, char *msg, size_t msg_len)
{
    Plan pl;
    if (msg && msg_len)
        msg[0] = 0;
    return check_and_plan(a, 0, &pl, msg, msg_len);
}

int qkv_epilogue_plan(const qkv_epilogue_args_t *a, qkv_epilogue_plan_t *plan)
{
    Plan pl;
    char msg[8];
    int rc = check_and_plan(a, 0, &pl, msg, sizeof msg);
    if (plan) {
        plan->vec_width = pl.W;
        plan->units_per_token = pl.U;
        plan->units_per_thread = pl.UPT;
        plan->block = kBlock;
        plan->grid = pl.grid;
        plan->lds_bytes = pl.lds;
    }
    return rc;
}

}  // extern "C"
