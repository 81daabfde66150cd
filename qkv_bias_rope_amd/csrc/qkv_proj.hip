// qkv_proj.hip -- the concat q|k|v projection with the epilogue in its output
// stage: y = x * W^T on the MFMA units (bf16 inputs, f32 accumulation), then
// bias, NeoX rotary embedding, write-back of the q/k/v rows and the K/V cache
// rows, all in one launch.
//
// The page "73 · D3-8 — G4 FusedQKV ported to CUDA" (§2, Excerpt C) feeds the
// epilogue from one matmul over the concat weight rows wq|wk|wv; here that
// matmul is a bf16 GEMM on gfx950's v_mfma_f32_32x32x16_bf16 and the epilogue
// runs on its accumulators instead of a second pass over HBM.
//
// Layout (verified on the GPU): for a 32x32x16 MFMA, lane l supplies
// A[l%32][8*(l/32) .. +8) and B[8*(l/32) .. +8)[l%32] (B[k][j] = W[j][k], so
// both operands are 16 contiguous bytes of a k-contiguous row) and receives
// D[8*(v/4) + 4*(l/32) + v%4][l%32], v < 16.
//
//  * Block tile 128 tokens x 256 outputs, four waves of 64 x 128; k tiles of
//    32 staged through double-buffered LDS (rows padded to 80 bytes so the
//    16-byte operand reads of 32 rows hit distinct banks).
//  * A wave's 128 output columns are one head (hd 128) or two (hd 64), so the
//    NeoX partner of column j (j + hd/2) sits in the same lane, in the MFMA
//    tile hd/64 tiles to the right: the rotation needs no data exchange.
//  * After the k loop the staging LDS holds a cos/sin table for the block's
//    128 tokens x hd/2 pair indices (double sincos rounded to f32, as in the
//    epilogue kernel).
//  * Decode (up to 4 tokens) is a weight-streaming GEMV, not a contraction
//    worth the matrix units: a separate kernel streams W with 16-byte loads,
//    reduces each dot product across the wave and runs the same epilogue.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "qkv_internal.h"

using namespace qkv_detail;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;        // tokens per block
constexpr int BN = 256;        // outputs per block
constexpr int BK = 32;         // k per stage
constexpr int ROWB = 80;       // LDS bytes per staged row (64 data + 16 pad)
constexpr int kThreads = 256;

struct ProjParams {
    const uint16_t *x;       // bf16 [nt][ld_x]
    const uint16_t *w;       // bf16 [N][K]
    int64_t ld_x;
    int K;                   // hidden
    int N;                   // nqt + 2*nkt
    int M;                   // nt
    int nqt, nkt, hd, half;
    float *out[3];           // q, k, v sections
    int64_t ld[3];
    const float *b[3];       // biases (may be null)
    const int32_t *pos;
    const int32_t *slot;
    void *cache[2];
    int64_t n_ctx, n_slots;
    unsigned int *err;
};

// cache row of token t, or -1 (and the error bit) when out of range
__device__ __forceinline__ int64_t cache_row(const ProjParams &p, int t)
{
    const int64_t ps = p.pos[t];
    const int64_t sl = p.slot ? (int64_t)p.slot[t] : 0;
    if (ps >= 0 && ps < p.n_ctx && sl >= 0 && sl < p.n_slots)
        return sl * p.n_ctx + ps;
    return -1;
}

__device__ __forceinline__ void rot(float &x0, float &x1, float c, float s)
{
    const double a = (double)x0, b = (double)x1, cd = (double)c, sd = (double)s;
    x0 = (float)(a * cd - b * sd);
    x1 = (float)(a * sd + b * cd);
}

template <bool F16>
__device__ __forceinline__ void put_cache(void *cache, int64_t off, float v)
{
    if constexpr (F16)
        static_cast<_Float16 *>(cache)[off] = static_cast<_Float16>(v);  // RNE
    else
        static_cast<float *>(cache)[off] = v;
}

// ---------------------------------------------------------------------------
// prefill / batched: MFMA GEMM + epilogue
// ---------------------------------------------------------------------------
template <bool F16, int HD>
__global__ __launch_bounds__(kThreads) void proj_mfma_kernel(ProjParams p, InvTable inv)
{
    extern __shared__ __align__(16) unsigned char lds[];
    // staging: two buffers of [BM + BN] rows x ROWB bytes
    constexpr int kStage = (BM + BN) * ROWB;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nblk = p.N / BN + (p.N % BN ? 1 : 0);
    const int n0 = ((int)blockIdx.x % nblk) * BN;
    const int m0 = ((int)blockIdx.x / nblk) * BM;

    // global -> register staging: A 128 rows x 4 chunks (2 per thread), B 256
    // rows x 4 chunks (4 per thread); out-of-range rows read a clamped row
    const int ch = tid & 3;
    int arow[2], brow[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        arow[j] = (tid >> 2) + 64 * j;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        brow[j] = (tid >> 2) + 64 * j;
    const uint16_t *ap[2], *bp[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        ap[j] = p.x + (int64_t)min(m0 + arow[j], p.M - 1) * p.ld_x + ch * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bp[j] = p.w + (int64_t)min(n0 + brow[j], p.N - 1) * p.K + ch * 8;

    u32x4 ra[2], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            ra[j] = *reinterpret_cast<const u32x4 *>(ap[j] + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            rb[j] = *reinterpret_cast<const u32x4 *>(bp[j] + k0);
    };
    auto lstore = [&](int buf) {
        unsigned char *s = lds + buf * kStage;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            *reinterpret_cast<u32x4 *>(s + arow[j] * ROWB + ch * 16) = ra[j];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4 *>(s + (BM + brow[j]) * ROWB + ch * 16) = rb[j];
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mi][ni][v] = 0.0f;

    const int KT = p.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int lr = lane & 31, lk = (lane >> 5) * 16;  // row in tile, byte offset of k chunk
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT)
            gload((kt + 1) * BK);
        const unsigned char *s = lds + (kt & 1) * kStage;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[2], b[4];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                a[mi] = *reinterpret_cast<const bf16x8 *>(
                    s + (wm * 64 + mi * 32 + lr) * ROWB + ks * 32 + lk);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                b[ni] = *reinterpret_cast<const bf16x8 *>(
                    s + (BM + wn * 128 + ni * 32 + lr) * ROWB + ks * 32 + lk);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < KT)
            lstore((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue --------------------------------------------------------
    constexpr int HALF = HD / 2;
    float *s_cos = reinterpret_cast<float *>(lds);
    float *s_sin = s_cos + BM * HALF;
    for (int e = tid; e < BM * HALF; e += kThreads) {
        const int r = e / HALF, i = e - (e / HALF) * HALF;
        const float a = (float)p.pos[min(m0 + r, p.M - 1)] * inv.v[i];
        double sd, cd;
        sincos((double)a, &sd, &cd);
        s_cos[e] = (float)cd;
        s_sin[e] = (float)sd;
    }
    __syncthreads();

    const int cw = n0 + wn * 128;  // first output column of this wave
    if (cw >= p.N)
        return;
    const int sec = cw < p.nqt ? 0 : (cw < p.nqt + p.nkt ? 1 : 2);
    const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
    float *const out = p.out[sec];
    const int64_t ldo = p.ld[sec];
    const float *const bias = p.b[sec];
    float bcol[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        bcol[ni] = bias ? bias[cw - sbase + ni * 32 + lr] : 0.0f;
    void *const cache = sec == 1 ? p.cache[0] : p.cache[1];

#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rt = wm * 64 + mi * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v & 3);
            const int t = m0 + rt;
            if (t >= p.M)
                continue;
            float y[4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                y[ni] = acc[mi][ni][v] + bcol[ni];   // f32 bias add
            if (sec < 2) {
                // pairs: tile ni with tile ni + HALF/32 inside each head
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int cih = (ni * 32) % HD;  // column of the tile inside its head
                    if (cih >= HALF)
                        continue;
                    const int nj = ni + HALF / 32;
                    const int i = cih + lr;          // pair index
                    rot(y[ni], y[nj], s_cos[rt * HALF + i], s_sin[rt * HALF + i]);
                }
            }
            const int64_t row = sec > 0 ? cache_row(p, t) : -1;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int c = cw - sbase + ni * 32 + lr;  // column inside the section
                out[(int64_t)t * ldo + c] = y[ni];
                if (row >= 0)
                    put_cache<F16>(cache, row * p.nkt + c, y[ni]);
            }
            if (sec > 0 && row < 0 && lr == 0)   // lanes 0 and 32 see every row
                atomicOr(p.err, 1u);
        }
    }
}

// ---------------------------------------------------------------------------
// decode (few tokens): weight-streaming GEMV + epilogue
// ---------------------------------------------------------------------------
// Block = 256 threads = 4 waves, 16 NeoX pairs = 32 output columns of one
// section (columns c0+j and c0+j+HALF, j < 16); each wave computes 8 columns
// for every token, a lane covering K/64 of each dot product.
constexpr int kGemvTok = 4;   // tokens per GEMV launch chunk

template <bool F16, int HD>
__global__ __launch_bounds__(kThreads) void proj_gemv_kernel(ProjParams p, InvTable inv, int t0)
{
    __shared__ float s_y[kGemvTok][32];
    constexpr int HALF = HD / 2;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // block -> (head, pair group): pair groups of 16 inside each head's HALF pairs
    const int groups = HALF / 16;
    const int head = (int)blockIdx.x / groups;
    const int g = (int)blockIdx.x - head * groups;
    const int hcol = head * HD;                 // first column of the head (global)
    const int nt = min(kGemvTok, p.M - t0);

    // this wave's 8 columns: local c in [wave*8, wave*8+8) of the block's 32;
    // local c < 16 -> column hcol + g*16 + c, else hcol + HALF + g*16 + (c-16)
    float dot[8][kGemvTok];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int tt = 0; tt < kGemvTok; ++tt)
            dot[j][tt] = 0.0f;
    int col[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = wave * 8 + j;
        col[j] = hcol + (c < 16 ? g * 16 + c : HALF + g * 16 + (c - 16));
    }
    for (int k0 = lane * 8; k0 < p.K; k0 += 64 * 8) {
        float xv[kGemvTok][8];
#pragma unroll
        for (int tt = 0; tt < kGemvTok; ++tt) {
            const u32x4 xr = *reinterpret_cast<const u32x4 *>(
                p.x + (int64_t)(t0 + min(tt, nt - 1)) * p.ld_x + k0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[tt][2 * e] = __uint_as_float(xr[e] << 16);
                xv[tt][2 * e + 1] = __uint_as_float(xr[e] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 wr = *reinterpret_cast<const u32x4 *>(p.w + (int64_t)col[j] * p.K + k0);
            float wv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                wv[2 * e] = __uint_as_float(wr[e] << 16);
                wv[2 * e + 1] = __uint_as_float(wr[e] & 0xffff0000u);
            }
#pragma unroll
            for (int tt = 0; tt < kGemvTok; ++tt)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dot[j][tt] = fmaf(xv[tt][e], wv[e], dot[j][tt]);
        }
    }
    // reduce across the wave
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int tt = 0; tt < kGemvTok; ++tt) {
            float v = dot[j][tt];
            for (int m = 32; m >= 1; m >>= 1)
                v += __shfl_xor(v, m, 64);
            dot[j][tt] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int tt = 0; tt < kGemvTok; ++tt)
                s_y[tt][wave * 8 + j] = dot[j][tt];
    }
    __syncthreads();

    // epilogue: thread (tt, j) for j < 16 handles the pair (j, j+16 of the block)
    const int tt = tid >> 4, j = tid & 15;
    if (tt >= nt)
        return;
    const int t = t0 + tt;
    const int sec = hcol < p.nqt ? 0 : (hcol < p.nqt + p.nkt ? 1 : 2);
    const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
    const int c0 = hcol - sbase + g * 16 + j;   // column inside the section
    const int c1 = c0 + HALF;
    const float *bias = p.b[sec];
    float y0 = s_y[tt][j] + (bias ? bias[c0] : 0.0f);
    float y1 = s_y[tt][16 + j] + (bias ? bias[c1] : 0.0f);
    if (sec < 2) {
        const float a = (float)p.pos[t] * inv.v[g * 16 + j];
        double sd, cd;
        sincos((double)a, &sd, &cd);
        rot(y0, y1, (float)cd, (float)sd);
    }
    float *out = p.out[sec];
    out[(int64_t)t * p.ld[sec] + c0] = y0;
    out[(int64_t)t * p.ld[sec] + c1] = y1;
    if (sec > 0) {
        const int64_t row = cache_row(p, t);
        void *cache = sec == 1 ? p.cache[0] : p.cache[1];
        if (row >= 0) {
            put_cache<F16>(cache, row * p.nkt + c0, y0);
            put_cache<F16>(cache, row * p.nkt + c1, y1);
        } else if (j == 0) {
            atomicOr(p.err, 1u);
        }
    }
}

template <bool F16, int HD>
hipError_t launch_proj(const ProjParams &pp, const InvTable &inv, hipStream_t st)
{
    if (pp.M <= kGemvTok) {
        // one block per 16 pairs of a head (the v section splits into heads too)
        const int blocks = (pp.N / HD) * (HD / 2 / 16);
        hipLaunchKernelGGL((proj_gemv_kernel<F16, HD>), dim3(blocks), dim3(kThreads), 0, st, pp,
                           inv, 0);
        return hipGetLastError();
    }
    const int nblk = pp.N / BN + (pp.N % BN ? 1 : 0);
    const int mblk = (pp.M + BM - 1) / BM;
    const int stage = 2 * (BM + BN) * ROWB;
    const int table = BM * (HD / 2) * 8;
    const int lds_bytes = stage > table ? stage : table;
    hipLaunchKernelGGL((proj_mfma_kernel<F16, HD>), dim3(nblk * mblk), dim3(kThreads),
                       (unsigned)lds_bytes, st, pp, inv);
    return hipGetLastError();
}

}  // namespace

extern "C" int qkv_epilogue_run_proj(qkv_epilogue_t *h, const qkv_proj_args_t *pa)
{
    if (!h)
        return QKV_ERR_INVALID_ARG;
    h->msg[0] = 0;
    if (!pa)
        return fail(h, QKV_ERR_INVALID_ARG, "args is NULL");
    const qkv_epilogue_args_t *a = &pa->epi;
    Plan pl;
    // the epilogue's checks, with the q/k/v sections as outputs and optional biases
    int rc = check_and_plan(a, h->n_ctx, &pl, h->msg, sizeof h->msg, kPlanBiasOptional);
    if (rc != QKV_OK)
        return rc;
    if (a->rope_style != QKV_ROPE_NEOX)
        return fail(h, QKV_ERR_UNSUPPORTED, "the projection path implements NeoX pairing only");
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(h, QKV_ERR_UNSUPPORTED, "the projection path needs head_dim 64 or 128, got %d",
                    a->head_dim);
    const int64_t N = pl.nqt + 2 * pl.nkt;
    if (pa->hidden <= 0 || pa->hidden % 32 != 0)
        return fail(h, QKV_ERR_INVALID_ARG, "hidden must be a positive multiple of 32, got %d",
                    pa->hidden);
    if (pl.nqt % 128 != 0 || pl.nkt % 128 != 0)
        return fail(h, QKV_ERR_UNSUPPORTED,
                    "the projection path needs q and k/v widths that are multiples of 128 "
                    "(got %lld and %lld)",
                    (long long)pl.nqt, (long long)pl.nkt);
    if (N > INT32_MAX / 2)
        return fail(h, QKV_ERR_INVALID_ARG, "q|k|v width too large");
    const int64_t ld_x = pa->ld_x ? pa->ld_x : pa->hidden;
    if (ld_x < pa->hidden || ld_x % 8 != 0)
        return fail(h, QKV_ERR_INVALID_ARG, "ld_x must be >= hidden and a multiple of 8");
    if (a->nt == 0)
        return QKV_OK;
    if (!pa->x || !pa->w || (uintptr_t)pa->x % 16 || (uintptr_t)pa->w % 16)
        return fail(h, QKV_ERR_INVALID_ARG, "x and w must be non-NULL and 16-byte aligned");
    {
        // x and w are read while the outputs are written: no byte in common
        // (hull test on each range, conservative for strided rows)
        const int64_t nt = a->nt, cb = a->cache_dtype == QKV_CACHE_F16 ? 2 : 4;
        const int64_t cache_bytes = pl.n_slots * pl.n_ctx * pl.nkt * cb;
        const uintptr_t ins[2][2] = {
            {(uintptr_t)pa->x, (uintptr_t)pa->x + (uintptr_t)(((nt - 1) * ld_x + pa->hidden) * 2)},
            {(uintptr_t)pa->w, (uintptr_t)pa->w + (uintptr_t)(N * pa->hidden * 2)}};
        const uintptr_t outs[5][2] = {
            {(uintptr_t)a->q, (uintptr_t)a->q + (uintptr_t)(((nt - 1) * pl.ld[0] + pl.nqt) * 4)},
            {(uintptr_t)a->k, (uintptr_t)a->k + (uintptr_t)(((nt - 1) * pl.ld[1] + pl.nkt) * 4)},
            {(uintptr_t)a->v, (uintptr_t)a->v + (uintptr_t)(((nt - 1) * pl.ld[2] + pl.nkt) * 4)},
            {(uintptr_t)a->kcache, (uintptr_t)a->kcache + (uintptr_t)cache_bytes},
            {(uintptr_t)a->vcache, (uintptr_t)a->vcache + (uintptr_t)cache_bytes}};
        const char *in_name[2] = {"x", "w"};
        const char *out_name[5] = {"q", "k", "v", "kcache", "vcache"};
        for (int i = 0; i < 2; ++i)
            for (int o = 0; o < 5; ++o)
                if (ins[i][0] < outs[o][1] && outs[o][0] < ins[i][1])
                    return fail(h, QKV_ERR_ALIAS, "read-only %s overlaps output %s", in_name[i],
                                out_name[o]);
    }

    ProjParams pp;
    pp.x = static_cast<const uint16_t *>(pa->x);
    pp.w = static_cast<const uint16_t *>(pa->w);
    pp.ld_x = ld_x;
    pp.K = pa->hidden;
    pp.N = (int)N;
    pp.M = a->nt;
    pp.nqt = (int)pl.nqt;
    pp.nkt = (int)pl.nkt;
    pp.hd = a->head_dim;
    pp.half = a->head_dim / 2;
    pp.out[0] = a->q;
    pp.out[1] = a->k;
    pp.out[2] = a->v;
    for (int s = 0; s < 3; ++s)
        pp.ld[s] = pl.ld[s];
    pp.b[0] = a->bq;
    pp.b[1] = a->bk;
    pp.b[2] = a->bv;
    pp.pos = a->pos;
    pp.slot = a->slot;
    pp.cache[0] = a->kcache;
    pp.cache[1] = a->vcache;
    pp.n_ctx = pl.n_ctx;
    pp.n_slots = pl.n_slots;
    pp.err = h->d_err;

    const InvTable &inv = handle_inv(h, a->theta, a->head_dim, a->freq_scale);
    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    const bool f16 = a->cache_dtype == QKV_CACHE_F16;
    if (a->head_dim == 128)
        e = f16 ? launch_proj<true, 128>(pp, inv, st) : launch_proj<false, 128>(pp, inv, st);
    else
        e = f16 ? launch_proj<true, 64>(pp, inv, st) : launch_proj<false, 64>(pp, inv, st);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    h->last_stream = st;
    return QKV_OK;
}
