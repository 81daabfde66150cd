// qkv_unfused.hip -- the unfused chain of the attention-input epilogue:
// add_bias x3, rope x2, store x2, seven launches per layer.
//
// This is the chain the fused kernel replaces (page "73 · D3-8 — G4 FusedQKV
// ported to CUDA", §1 and §2: per layer three bias adds, two rope launches and
// two KV stores, each a sub-2 us kernel).  It exists for the same-binary A/B
// the page measures (§5: launches per decode step, wall clock with and without
// the fusion) and as a second GPU implementation the fused kernel must match
// bit for bit (both rotary styles, any frequency scale).  Each kernel keeps
// the numerics of the fused kernel (one f32 bias add; f32 angle, cos/sin in
// double rounded to f32; rotation in double; binary16 round-to-nearest-even
// stores) but, like the page's unfused rope, every rope thread evaluates
// cos/sin for its own pairs.

#include <hip/hip_runtime.h>

#include <cstring>

#include "qkv_internal.h"

using namespace qkv_detail;

namespace {

constexpr int kBlockU = 256;

// x[t][c..c+W) += b[c..c+W) over nt rows of `width` elements (stride ld).
template <int W, bool STREAM>
__global__ __launch_bounds__(kBlockU) void add_bias_kernel(float *x, int64_t ld,
                                                           const float *b, int width,
                                                           int64_t n_items)
{
    const int64_t g = (int64_t)blockIdx.x * kBlockU + threadIdx.x;
    if (g >= n_items)
        return;
    const int per_row = width / W;
    const int64_t t = g / per_row;
    const int c = (int)(g - t * per_row) * W;
    float *p = x + t * ld + c;
    FVec<W> v = ld_data<W, STREAM>(p);
    const FVec<W> bv = ld_vec<W>(b + c);
#pragma unroll
    for (int e = 0; e < W; ++e)
        v.e[e] = v.e[e] + bv.e[e];
    st_data<W, STREAM>(p, v);
}

// Turn (x0, x1) by the f32 angle a: cos/sin in double rounded to f32, the
// rotation in double.
__device__ __forceinline__ void turn(float &x0, float &x1, float a)
{
    double sd, cd;
    sincos((double)a, &sd, &cd);
    const double c = (double)(float)cd;
    const double s = (double)(float)sd;
    const double u = (double)x0, w = (double)x1;
    x0 = (float)(u * c - w * s);
    x1 = (float)(u * s + w * c);
}

// Rotation of n_heads heads per row; item (t, h, m) owns the slots
// [eo, eo+W) and [eo+d, eo+d+W) of head h, eo = m*W.
//  NeoX (STYLE 0): d = half; element eo+e pairs with eo+e+half, angle index
//    eo+e.
//  interleaved (STYLE 1): W = 4: d = half, each slot holds W/2 adjacent pairs
//    (pair indices eo/2 + j and (eo+half)/2 + j); W = 1: the slots are
//    x[2m] and x[2m+1], pair index m.
template <int W, bool STREAM, int STYLE, typename TAB>
__global__ __launch_bounds__(kBlockU) void rope_kernel(float *x, int64_t ld, int n_heads,
                                                       int hd, const int32_t *pos,
                                                       TAB inv, int64_t n_items)
{
    const int64_t g = (int64_t)blockIdx.x * kBlockU + threadIdx.x;
    if (g >= n_items)
        return;
    const int half = hd / 2;
    const int per_head = half / W;
    const int64_t per_row = (int64_t)n_heads * per_head;
    const int64_t t = g / per_row;
    const int r = (int)(g - t * per_row);
    const int h = r / per_head;
    const int m = r - h * per_head;
    const bool adj1 = STYLE == 1 && W == 1;
    const int eo = adj1 ? 2 * m : m * W;
    const int d = adj1 ? 1 : half;
    float *p = x + t * ld + (int64_t)h * hd + eo;
    FVec<W> xa = ld_data<W, STREAM>(p);
    FVec<W> xb = ld_data<W, STREAM>(p + d);
    const float pf = (float)pos[t];
    if constexpr (STYLE == 0) {
#pragma unroll
        for (int e = 0; e < W; ++e)
            turn(xa.e[e], xb.e[e], pf * inv.v[eo + e]);   // f32 angle
    } else if constexpr (W == 1) {
        turn(xa.e[0], xb.e[0], pf * inv.v[m]);
    } else {
#pragma unroll
        for (int j = 0; j < W / 2; ++j) {
            turn(xa.e[2 * j], xa.e[2 * j + 1], pf * inv.v[eo / 2 + j]);
            turn(xb.e[2 * j], xb.e[2 * j + 1], pf * inv.v[(eo + half) / 2 + j]);
        }
    }
    st_data<W, STREAM>(p, xa);
    st_data<W, STREAM>(p + d, xb);
}

// cache[row(t)][c..c+W) = cvt(x[t][c..c+W)), row = slot*n_ctx + pos; a token
// whose position or slot is out of range writes nothing and sets the error
// word.
template <int W, bool F16, bool STREAM>
__global__ __launch_bounds__(kBlockU) void store_kernel(const float *x, int64_t ld, int nkt,
                                                        const int32_t *pos, const int32_t *slot,
                                                        int64_t n_ctx, int64_t n_slots,
                                                        void *cache, unsigned int *err,
                                                        int64_t n_items)
{
    const int64_t g = (int64_t)blockIdx.x * kBlockU + threadIdx.x;
    if (g >= n_items)
        return;
    const int per_row = nkt / W;
    const int64_t t = g / per_row;
    const int c = (int)(g - t * per_row) * W;
    const int64_t ps = pos[t];
    const int64_t sl = slot ? (int64_t)slot[t] : 0;
    if (ps < 0 || ps >= n_ctx || sl < 0 || sl >= n_slots) {
        if (c == 0)
            atomicOr(err, 1u);
        return;
    }
    const FVec<W> v = ld_data<W, STREAM>(x + t * ld + c);
    st_cache<W, F16, STREAM>(cache, (sl * n_ctx + ps) * nkt + c, v);
}

unsigned grid_of(int64_t n_items)
{
    return (unsigned)((n_items + kBlockU - 1) / kBlockU);
}

template <int W, bool F16, bool STREAM, int STYLE, typename TAB>
hipError_t launch_chain(const qkv_epilogue_args_t *a, const Plan &pl, const TAB &inv,
                        unsigned int *err, hipStream_t st)
{
    const int64_t nt = a->nt;
    const int nqt = (int)pl.nqt, nkt = (int)pl.nkt;
    float *xs[3] = {a->q, a->k, a->v};
    const float *bs[3] = {a->bq, a->bk, a->bv};
    const int widths[3] = {nqt, nkt, nkt};
    // add_bias x3
    for (int s = 0; s < 3; ++s) {
        const int64_t n = nt * (widths[s] / W);
        hipLaunchKernelGGL((add_bias_kernel<W, STREAM>), dim3(grid_of(n)), dim3(kBlockU), 0, st,
                           xs[s], pl.ld[s], bs[s], widths[s], n);
    }
    // rope x2
    const int heads[2] = {a->n_head, a->n_kv_head};
    for (int s = 0; s < 2; ++s) {
        const int64_t n = nt * heads[s] * (pl.half / W);
        hipLaunchKernelGGL((rope_kernel<W, STREAM, STYLE, TAB>), dim3(grid_of(n)), dim3(kBlockU), 0, st,
                           xs[s], pl.ld[s], heads[s], a->head_dim, a->pos, inv, n);
    }
    // store x2 (K from the k section, V from the v section)
    void *caches[2] = {a->kcache, a->vcache};
    for (int s = 0; s < 2; ++s) {
        const int64_t n = nt * (nkt / W);
        hipLaunchKernelGGL((store_kernel<W, F16, STREAM>), dim3(grid_of(n)), dim3(kBlockU), 0, st,
                           (const float *)xs[s + 1], pl.ld[s + 1], nkt, a->pos, a->slot, pl.n_ctx,
                           pl.n_slots, caches[s], err, n);
    }
    return hipGetLastError();
}

template <int W, typename TAB>
hipError_t launch_chain_w(const qkv_epilogue_args_t *a, const Plan &pl, const TAB &inv,
                          unsigned int *err, hipStream_t st)
{
    const bool f16 = a->cache_dtype == QKV_CACHE_F16;
    const bool il = pl.style == QKV_ROPE_INTERLEAVED;
    if (pl.stream) {
        if (il)
            return f16 ? launch_chain<W, true, true, 1>(a, pl, inv, err, st)
                       : launch_chain<W, false, true, 1>(a, pl, inv, err, st);
        return f16 ? launch_chain<W, true, true, 0>(a, pl, inv, err, st)
                   : launch_chain<W, false, true, 0>(a, pl, inv, err, st);
    }
    if (il)
        return f16 ? launch_chain<W, true, false, 1>(a, pl, inv, err, st)
                   : launch_chain<W, false, false, 1>(a, pl, inv, err, st);
    return f16 ? launch_chain<W, true, false, 0>(a, pl, inv, err, st)
               : launch_chain<W, false, false, 0>(a, pl, inv, err, st);
}

}  // namespace

extern "C" int qkv_epilogue_run_unfused(qkv_epilogue_t *h, const qkv_epilogue_args_t *a)
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
    const InvTable &inv = handle_inv(h, a->theta, a->head_dim, a->freq_scale);
    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    if (pl.half <= kSmallHalf) {
        const InvTableSmall sm = small_table(inv);
        e = pl.W == 4 ? launch_chain_w<4>(a, pl, sm, h->d_err, st)
                      : launch_chain_w<1>(a, pl, sm, h->d_err, st);
    } else {
        e = pl.W == 4 ? launch_chain_w<4>(a, pl, inv, h->d_err, st)
                      : launch_chain_w<1>(a, pl, inv, h->d_err, st);
    }
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return QKV_OK;
}
