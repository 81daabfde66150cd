// qkv_host.cpp -- the host-only part of libqkv_epilogue.so: argument
// validation, the launch planner and the inverse-frequency tables, and the
// four C entry points that run nothing on a device (qkv_epilogue_check_args,
// qkv_epilogue_plan, qkv_epilogue_inv_freq, qkv_epilogue_inv_freq_scaled).
// Plain C++ with no HIP dependency, so that it also builds with a host
// compiler alone (the sanitizer build of the tests).
//
// The checks are those run_ex documents in include/qkv_epilogue.h; the
// inverse frequencies are theta^(-2i/head_dim) of page "73 · D3-8 — G4
// FusedQKV ported to CUDA" §3.2 Excerpt A, computed in double and rounded
// once to f32.

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "qkv_plan.h"

namespace qkv_detail {

int ceil_div(int64_t a, int64_t b)
{
    return (int)((a + b - 1) / b);
}

// Tiling of the (token x unit) space, one unit per thread.  Measured on
// MI355X (14B shape, 896 units per token, kernel time from HIP-graph replays
// over rotating input sets):
//  * thousands of tokens (prefill): 128-thread column blocks, one token per
//    workgroup, nontemporal data (the launch streams far more than the
//    caches hold) -- the per-workgroup cos/sin (64 values) rides under the
//    load latency;
//  * hundreds of tokens (batched decode): 256-thread column blocks, one
//    token per workgroup (256 sequences: 4.6 us, against 4.7-4.9 us for
//    64-896 threads and 4.9-7.4 us for two or four tokens per workgroup);
//  * a few tokens (decode): 64-thread blocks spread one token over many
//    workgroups, default cache policy (the data is cache-resident).
void choose_tiling(int64_t nt, int U, int uph, Plan *pl)
{
    if (nt >= 1024) {
        pl->nthr = 128;
        pl->tb = 1;
        pl->stream = true;
    } else if (nt >= 64) {
        pl->nthr = ceil_div(U, 64) * 64;
        if (pl->nthr > 256)
            pl->nthr = 256;
        pl->tb = 1;
        pl->stream = true;
    } else {
        pl->nthr = 64;
        pl->tb = 1;
        pl->stream = false;
    }
    if (pl->norm) {
        // whole heads per column block: a multiple of the units per head
        int k = (pl->nthr + uph / 2) / uph;
        k = k < 1 ? 1 : k;
        while (k > 1 && k * uph > kMaxBlock)
            --k;
        pl->nthr = k * uph;
    }
    pl->ncb = ceil_div(U, pl->nthr);
}

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
                   size_t mlen, unsigned flags, const float *wq, const float *wk, float eps)
{
    if (!a) {
        set_msg(msg, mlen, "args is NULL");
        return QKV_ERR_INVALID_ARG;
    }
    if (a->rope_style != QKV_ROPE_NEOX && a->rope_style != QKV_ROPE_INTERLEAVED) {
        set_msg(msg, mlen,
                "rope_style %d not supported: NeoX pairing (i, i+head_dim/2) = 0 and "
                "interleaved pairing (2i, 2i+1) = 1 are implemented",
                a->rope_style);
        return QKV_ERR_UNSUPPORTED;
    }
    if (a->freq_scale != 0.0f && (!(a->freq_scale > 0.0f) || !std::isfinite(a->freq_scale))) {
        set_msg(msg, mlen, "freq_scale must be finite and > 0 (0 means 1), got %g",
                (double)a->freq_scale);
        return QKV_ERR_INVALID_ARG;
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
    pl->stream = false;
    pl->norm = (flags & kPlanNorm) != 0;
    pl->style = a->rope_style;
    pl->nthr = 64;
    pl->ncb = 1;
    pl->tb = 1;
    pl->grid = 0;
    pl->lds = 0;

    if (a->nt == 0)
        return QKV_OK;

    const bool bias_opt = (flags & kPlanBiasOptional) != 0;
    struct {
        const void *p;
        const char *n;
        bool optional;
    } ptrs[] = {{a->q, "q", false},          {a->k, "k", false},
                {a->v, "v", false},          {a->bq, "bq", bias_opt},
                {a->bk, "bk", bias_opt},     {a->bv, "bv", bias_opt},
                {a->pos, "pos", false},      {a->kcache, "kcache", false},
                {a->vcache, "vcache", false}};
    for (auto &e : ptrs) {
        if (!e.p && !e.optional) {
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
    if (flags & kPlanNorm) {
        if (!wq || !wk) {
            set_msg(msg, mlen, "%s is NULL", wq ? "w_k" : "w_q");
            return QKV_ERR_INVALID_ARG;
        }
        if ((uintptr_t)wq % 4 || (uintptr_t)wk % 4) {
            set_msg(msg, mlen, "norm weight pointer not 4-byte aligned");
            return QKV_ERR_INVALID_ARG;
        }
        if (!(eps >= 0.0f) || !std::isfinite(eps)) {
            set_msg(msg, mlen, "norm eps must be finite and >= 0, got %g", (double)eps);
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
    const int64_t wbytes = (flags & kPlanNorm) ? (int64_t)a->head_dim * 4 : 0;
    Span ins[7] = {
        {(uintptr_t)a->bq, 0, a->bq ? nqt * 4 : 0, 1, "bq"},
        {(uintptr_t)a->bk, 0, a->bk ? nkt * 4 : 0, 1, "bk"},
        {(uintptr_t)a->bv, 0, a->bv ? nkt * 4 : 0, 1, "bv"},
        {(uintptr_t)a->pos, 0, nt * 4, 1, "pos"},
        {(uintptr_t)a->slot, 0, a->slot ? nt * 4 : 0, 1, "slot"},
        {(uintptr_t)wq, 0, wbytes, 1, "w_q"},
        {(uintptr_t)wk, 0, wbytes, 1, "w_k"},
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
        vec = vec && ((uintptr_t)f % 16) == 0;  // NULL (no bias) is aligned
    vec = vec && ((uintptr_t)wq % 16) == 0 && ((uintptr_t)wk % 16) == 0;
    vec = vec && (ldq % 4) == 0 && (ldk % 4) == 0 && (ldv % 4) == 0;
    vec = vec && ((uintptr_t)a->kcache % (4 * cb)) == 0 && ((uintptr_t)a->vcache % (4 * cb)) == 0;
    const int W = vec ? 4 : 1;
    const int half = a->head_dim / 2;
    const int64_t U = (int64_t)(a->n_head + a->n_kv_head) * (half / W) + nkt / (2 * W);
    if (U >= (1 << 22)) {
        set_msg(msg, mlen, "rows too wide: %lld work units per token (at most %d)", (long long)U,
                (1 << 22) - 1);
        return QKV_ERR_INVALID_ARG;
    }
    pl->W = W;
    pl->U = (int)U;
    choose_tiling(nt, (int)U, half / W, pl);
    const int64_t ntb = (nt + pl->tb - 1) / pl->tb;
    pl->grid = ntb * pl->ncb;
    if (pl->grid > INT32_MAX) {
        set_msg(msg, mlen, "launch too large: %lld workgroups (split the tokens)", (long long)pl->grid);
        return QKV_ERR_INVALID_ARG;
    }
    pl->lds = lds_row_bytes(pl->tb) + 2 * pl->tb * half * 4;  // <= 2 KB + 16 for one token
    if (pl->norm)
        pl->lds += pl->tb * pl->nthr * 8;  // per-lane partial sums of squares
    return QKV_OK;
}

void host_inv_freq(float theta, int head_dim, float freq_scale, float *out)
{
    const int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        const double f = std::pow((double)theta, -(double)(2 * i) / (double)head_dim);
        out[i] = freq_scale == 1.0f ? (float)f : (float)((double)freq_scale * f);
    }
}

}  // namespace qkv_detail

using namespace qkv_detail;

extern "C" {

int qkv_epilogue_inv_freq(float theta, int head_dim, float *out)
{
    if (!out || head_dim <= 0 || (head_dim & 1) || head_dim > QKV_MAX_HEAD_DIM ||
        !(theta > 0.0f) || !std::isfinite(theta))
        return QKV_ERR_INVALID_ARG;
    host_inv_freq(theta, head_dim, 1.0f, out);
    return QKV_OK;
}

int qkv_epilogue_inv_freq_scaled(float theta, float freq_scale, int head_dim, float *out)
{
    if (!out || head_dim <= 0 || (head_dim & 1) || head_dim > QKV_MAX_HEAD_DIM ||
        !(theta > 0.0f) || !std::isfinite(theta) || !(freq_scale > 0.0f) ||
        !std::isfinite(freq_scale))
        return QKV_ERR_INVALID_ARG;
    host_inv_freq(theta, head_dim, freq_scale, out);
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
        plan->units_per_thread = 1;
        plan->block = pl.nthr;
        plan->col_blocks = pl.ncb;
        plan->tokens_per_block = pl.tb;
        plan->grid = pl.grid;
        plan->lds_bytes = pl.lds;
    }
    return rc;
}

}  // extern "C"
