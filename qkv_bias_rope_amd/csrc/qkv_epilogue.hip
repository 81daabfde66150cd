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
//    unit is [c, c+W) and [c+nkt/2, c+nkt/2+W), so that, like the rope
//    units, consecutive lanes touch consecutive 16 bytes and every store
//    instruction writes whole 128-byte lines.  Units of a token are ordered
//    q, k, v.
//  * Grid.  A workgroup owns a column block (a fixed range of units) and a
//    token block.  Each thread decodes its units once, keeps their biases in
//    registers and walks the tokens of its block, issuing the next token's
//    loads before it computes the current one.  Prefill and batched decode
//    pick few, wide column blocks and several tokens per block; a one-token
//    decode spreads the token over many small column blocks.
//  * cos/sin are computed once per (token, pair index) per workgroup, in double
//    precision, rounded to f32 and kept in LDS; the inverse frequencies ride in
//    the kernel arguments (computed on the host once per theta/head_dim).
//  * The rotation is evaluated in double: the products of two f32 values are
//    exact in double, so x0*c - x1*s is rounded once there and once to f32
//    whether or not the compiler fuses it into an FMA.
//  * q/k/v and the cache rows are touched exactly once per launch, so their
//    loads and stores carry the nontemporal hint; the biases (reused by every
//    workgroup) do not.
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

#include "qkv_internal.h"

using namespace qkv_detail;

namespace {

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
    uint64_t uph_mul;     // ceil(2^40 / uph): n / uph == (n * uph_mul) >> 40 for n < 2^22
    uint64_t half_mul;    // ceil(2^40 / half), the same for half
    int nt;
    int hd;
    int half;
    int uph;              // rope units per head = half / W
    int qu;               // q rope units per token
    int qku;              // q + k rope units per token
    int vhalf;            // nkt / 2: distance between the two slots of a v unit
    int U;                // units per token
    int cbu;              // units per column block = blockDim.x
    int tb;               // tokens per token block
    unsigned has_bias;    // bit s: section s has a bias (all set for run/run_ex)
    const float *nw[2];   // q/k norm weights [hd] (q/k-norm variant only)
    double eps;           // q/k norm epsilon
};

// n / d for 0 <= n < 2^22 and 1 <= d <= 256 with mul = ceil(2^40 / d): the
// product overestimates n/d by less than 2^-18, and the fraction of n/d is at
// most 1 - 1/d, so the floor is exact.  Replaces a runtime integer division
// (a few dozen instructions) in front of the data loads.
__device__ __forceinline__ int div_small(int n, uint64_t mul)
{
    return (int)(((uint64_t)(uint32_t)n * mul) >> 40);
}

// Unit r of a token (0 <= r < U): section, column of the first slot, offset
// of the first slot inside its head (rope units), index of the unit inside
// its head, and distance from the first slot to the second.  Written with
// selects only, so that nothing branches before the data loads are issued.
//  NeoX (STYLE 0):   slots [eo, eo+W) and [eo+half, ...), eo = m*W; element
//                    eo+e of the first slot pairs with element eo+e+half.
//  interleaved (1):  W = 4: the same slots, each holding W/2 adjacent pairs
//                    (2j, 2j+1); W = 1: the slots are x[2m] and x[2m+1].
template <int W, int STYLE>
__device__ __forceinline__ void decode_unit(const KParams &p, int r, int &sec, int &col, int &eo,
                                            int &m, int &d1)
{
    const bool rope = r < p.qku;
    sec = rope ? (r < p.qu ? 0 : 1) : 2;
    const int rr = r - (sec == 1 ? p.qu : 0);  // unit index inside the q or k section
    const int h = div_small(rr, p.uph_mul);
    const int mm = rr - h * p.uph;
    constexpr bool adj = STYLE == 1 && W == 1;  // scalar interleaved: slots 2m, 2m+1
    const int e = adj ? 2 * mm : mm * W;
    eo = rope ? e : 0;
    m = rope ? mm : 0;
    col = rope ? h * p.hd + e : (r - p.qku) * W;
    d1 = rope ? (adj ? 1 : p.half) : p.vhalf;
}

// (x0, x1) -> (x0*c - x1*s, x0*s + x1*c), evaluated in double: the products of
// two f32 values are exact there, so each result is rounded once in double
// and once to f32 whether or not the compiler fuses it into an FMA.
__device__ __forceinline__ void rotate_pair(float &x0, float &x1, float c, float s)
{
    const double a = (double)x0, b = (double)x1, cd = (double)c, sd = (double)s;
    x0 = (float)(a * cd - b * sd);
    x1 = (float)(a * sd + b * cd);
}

// A 64-bit value that is the same in every active lane, as a scalar.
__device__ __forceinline__ int64_t readfirstlane64(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Cache row of a token: slot*n_ctx + pos (slot 0 without slots), or -1 with
// the error bit set when the position or the slot is out of range (the token
// then writes no cache row).
__device__ __forceinline__ int64_t cache_row(const KParams &p, int32_t pos, int32_t slot_or_pos)
{
    const int64_t sl = p.slot ? (int64_t)slot_or_pos : 0;
    if (pos >= 0 && (int64_t)pos < p.n_ctx && sl >= 0 && sl < p.n_slots)
        return sl * p.n_ctx + pos;
    atomicOr(p.err, 1u);
    return -1;
}

// Section operands picked with selects on wave-uniform kernel arguments (an
// indexed read of the argument array would become a per-lane memory load in
// front of every data load).
template <typename T>
__device__ __forceinline__ T pick3(int s, T a, T b, T c)
{
    return s == 0 ? a : (s == 1 ? b : c);
}

// NORM: the q/k-norm variant -- after the bias, every q and k head is scaled
// by w / sqrt(mean(x^2) + eps) before the rotation.  The sum of squares is
// taken in double (exact squares), each lane adding its 2W elements first.
//   NORM == 1: lanes write their partials to LDS before the barrier and every
//              lane of a head sums the head's partials in the same order
//              (any units-per-head count);
//   NORM == 2: the units per head are a power of two dividing 64, so a head's
//              lanes are aligned inside one wave and an xor butterfly gives
//              every lane of the head the same sum (addition is commutative)
//              with no LDS and no wait at the barrier.
// Column blocks hold whole heads (the planner makes blockDim a multiple of the
// units per head).
template <int W, bool F16, int TPB, bool STREAM, int NORM, int STYLE, typename TAB>
__global__ __launch_bounds__(kMaxBlock) void qkv_epilogue_kernel(KParams p, TAB inv)
{
    extern __shared__ __align__(16) unsigned char lds_raw[];
    int64_t *s_row = reinterpret_cast<int64_t *>(lds_raw);
    float *s_cos = reinterpret_cast<float *>(lds_raw + lds_row_bytes(TPB));
    float *s_sin = s_cos + TPB * p.half;
    double *s_ss = reinterpret_cast<double *>(s_sin + TPB * p.half);  // NORM: [TPB][nthr]

    // The kernel arguments the data addresses depend on, fetched in one batch
    // of scalar loads: an empty asm that takes them as scalar-register inputs
    // keeps the compiler from issuing them in several rounds next to their
    // first uses, each round a wait on the scalar cache before the data
    // loads can go out.
    asm volatile("" ::"s"(p.x[0]), "s"(p.x[1]), "s"(p.x[2]), "s"(p.b[0]), "s"(p.b[1]), "s"(p.b[2]),
                 "s"(p.pos), "s"(p.slot), "s"(p.ld[0]), "s"(p.ld[1]), "s"(p.ld[2]), "s"(p.uph_mul),
                 "s"(p.half_mul), "s"(p.nt), "s"(p.hd), "s"(p.half), "s"(p.uph), "s"(p.qu),
                 "s"(p.qku), "s"(p.vhalf), "s"(p.U), "s"(p.cbu), "s"(p.has_bias), "s"(gridDim.y));
    const int tid = (int)threadIdx.x;
    const int nthr = (int)blockDim.x;
    // grid: x = column block, (y, z) = token block (z only past 65535 blocks)
    const int cb = (int)blockIdx.x;
    const int64_t tb0 = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * TPB;
    if (tb0 >= p.nt)
        return;  // the tail of the last z slice (uniform over the workgroup)
    const int t0 = (int)tb0;
    const int ntok = min(TPB, p.nt - t0);
    const int ent = ntok * p.half;

    // Every load below is unconditional (out-of-range lanes read a clamped,
    // valid address and discard it) so that each wait covers exactly the
    // loads it needs: the cos/sin inputs are loaded first and their wait does
    // not hold up the data loads issued after them.

    // ---- cos/sin input of this thread's first entry ------------------------
    // Entry e = tk*half + i is (token tk, pair index i); the lane of entry
    // (tk, 0) also forms token tk's cache row, from the position it already
    // holds.  These loads take per-lane indices, so none of them is turned
    // into a scalar value the compiler would wait for before the data loads.
    const int ec = min(tid, ent - 1);
    const int e_tk = div_small(ec, p.half_mul);
    const int e_i = ec - e_tk * p.half;
    const int32_t e_pos = p.pos[t0 + e_tk];
    const int32_t e_slot = (p.slot ? p.slot : p.pos)[t0 + e_tk];
    const float e_inv = inv.v[e_i];

    // ---- this thread's unit, its biases and its data for every token -------
    const int r = cb * p.cbu + tid;
    const bool live = r < p.U;
    int sec, col, i0, m, d1;
    decode_unit<W, STYLE>(p, min(r, p.U - 1), sec, col, i0, m, d1);
    float *const xsec = pick3(sec, p.x[0], p.x[1], p.x[2]);
    float *const xs = xsec + col;
    const int64_t ldx = pick3(sec, p.ld[0], p.ld[1], p.ld[2]);
    // A section without a bias reads its own first row instead (a valid
    // address; the values are replaced by zero below) -- no branch, so the
    // waits stay exact.
    const bool hb = (p.has_bias >> sec) & 1u;
    const float *const bp = hb ? pick3(sec, p.b[0], p.b[1], p.b[2]) + col : xs;
    FVec<W> ba = ld_vec<W>(bp);
    FVec<W> bb = ld_vec<W>(bp + d1);
    FVec<W> wa, wb;
    if constexpr (NORM != 0) {
        // weights of the pair indices of this unit; v units read q's (unused)
        const float *wp = (sec == 1 ? p.nw[1] : p.nw[0]) + i0;
        wa = ld_vec<W>(wp);
        wb = ld_vec<W>(wp + (sec < 2 ? d1 : 0));
    }
    FVec<W> xa[TPB], xb[TPB];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
        const float *xp = xs + (int64_t)(t0 + min(tt, ntok - 1)) * ldx;
        xa[tt] = ld_data<W, STREAM>(xp);
        xb[tt] = ld_data<W, STREAM>(xp + d1);
    }

    // ---- cos/sin per (token, pair index) and cache row per token -----------
    if (tid < ent) {
        const float a = (float)e_pos * e_inv;   // f32 angle
        double sd, cd;
        sincos((double)a, &sd, &cd);
        s_cos[tid] = (float)cd;
        s_sin[tid] = (float)sd;
        if (e_i == 0)
            s_row[e_tk] = cache_row(p, e_pos, e_slot);
    }
    for (int e = tid + nthr; e < ent; e += nthr) {  // only when TPB*half > nthr
        const int tk = div_small(e, p.half_mul);
        const int i = e - tk * p.half;
        const int32_t ps = p.pos[t0 + tk];
        const float a = (float)ps * inv.v[i];
        double sd, cd;
        sincos((double)a, &sd, &cd);
        s_cos[e] = (float)cd;
        s_sin[e] = (float)sd;
        if (i == 0)
            s_row[tk] = cache_row(p, ps, (p.slot ? p.slot : p.pos)[t0 + tk]);
    }
#pragma unroll
    for (int e = 0; e < W; ++e) {
        ba.e[e] = hb ? ba.e[e] : 0.0f;
        bb.e[e] = hb ? bb.e[e] : 0.0f;
    }
    if constexpr (NORM == 1) {
        // this lane's part of its head's sum of squares, per token
#pragma unroll
        for (int tt = 0; tt < TPB; ++tt) {
            double ss = 0.0;
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const double xa0 = (double)(xa[tt].e[e] + ba.e[e]);
                const double xb0 = (double)(xb[tt].e[e] + bb.e[e]);
                ss += xa0 * xa0;
                ss += xb0 * xb0;
            }
            s_ss[tt * nthr + tid] = ss;
        }
    }
    __syncthreads();
    if (!live)
        return;

    // ---- bias, rotate, write back, store the cache rows --------------------
    void *const cache = sec == 1 ? p.cache[0] : p.cache[1];
#pragma unroll
    for (int tt = 0; tt < TPB; ++tt) {
        if (tt >= ntok)
            break;
        FVec<W> ra, rb;
#pragma unroll
        for (int e = 0; e < W; ++e) {
            ra.e[e] = xa[tt].e[e] + ba.e[e];
            rb.e[e] = xb[tt].e[e] + bb.e[e];
        }
        if constexpr (NORM == 2) {
            // butterfly over the head's lanes (all lanes take part: v lanes
            // sit in groups of their own and their sums are not used)
            double ss = 0.0;
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const double xa0 = (double)ra.e[e];
                const double xb0 = (double)rb.e[e];
                ss += xa0 * xa0;
                ss += xb0 * xb0;
            }
            for (int m = p.uph >> 1; m >= 1; m >>= 1)
                ss += __shfl_xor(ss, m, 64);
            if (sec < 2) {
                const double rr = 1.0 / sqrt(ss / (double)p.hd + p.eps);
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    ra.e[e] = (float)((double)ra.e[e] * rr * (double)wa.e[e]);
                    rb.e[e] = (float)((double)rb.e[e] * rr * (double)wb.e[e]);
                }
            }
        }
        if (sec < 2) {
            if constexpr (NORM == 1) {
                // sum of the head's partials, in unit order (same for every lane)
                const double *hp = s_ss + tt * nthr + (tid - m);
                double ss = 0.0;
                for (int j = 0; j < p.uph; ++j)
                    ss += hp[j];
                const double rr = 1.0 / sqrt(ss / (double)p.hd + p.eps);
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    ra.e[e] = (float)((double)ra.e[e] * rr * (double)wa.e[e]);
                    rb.e[e] = (float)((double)rb.e[e] * rr * (double)wb.e[e]);
                }
            }
            if constexpr (STYLE == 0) {
                const int ci = tt * p.half + i0;
                const FVec<W> cs = ld_vec<W>(s_cos + ci);
                const FVec<W> sn = ld_vec<W>(s_sin + ci);
#pragma unroll
                for (int e = 0; e < W; ++e)
                    rotate_pair(ra.e[e], rb.e[e], cs.e[e], sn.e[e]);
            } else if constexpr (W == 1) {
                const int ci = tt * p.half + m;
                rotate_pair(ra.e[0], rb.e[0], s_cos[ci], s_sin[ci]);
            } else {
                // adjacent pairs inside each slot: pair indices eo/2 + j and
                // (eo + half)/2 + j, j < W/2
                const int ca = tt * p.half + i0 / 2;
                const int cb2 = ca + p.half / 2;
#pragma unroll
                for (int j = 0; j < W / 2; ++j) {
                    rotate_pair(ra.e[2 * j], ra.e[2 * j + 1], s_cos[ca + j], s_sin[ca + j]);
                    rotate_pair(rb.e[2 * j], rb.e[2 * j + 1], s_cos[cb2 + j], s_sin[cb2 + j]);
                }
            }
        }
        const int64_t row = s_row[tt];
        if constexpr (STREAM) {
            // The bases of the stores are this token's row of the lane's
            // section and its cache row.  When every lane of the wave works on
            // one section (always, when the sections' unit counts are
            // multiples of 64), they are taken from the first lane: the buffer
            // resource is then a scalar value and each store one instruction.
            // A wave spanning two sections takes the per-lane bases, and the
            // compiler loops over their distinct values.
            const int sec0 = __builtin_amdgcn_readfirstlane(sec);
            if (__builtin_amdgcn_ballot_w64(sec != sec0) == 0) {
                const int64_t tok = t0 + tt;
                float *const xrow = pick3(sec0, p.x[0], p.x[1], p.x[2]) +
                                    tok * pick3(sec0, p.ld[0], p.ld[1], p.ld[2]);
                st_stream<W>(xrow, (uint32_t)col * 4u, ra);
                st_stream<W>(xrow, (uint32_t)(col + d1) * 4u, rb);
                const int64_t row0 = readfirstlane64(row);
                if (sec0 > 0 && row0 >= 0) {
                    void *const crow = static_cast<char *>(sec0 == 1 ? p.cache[0] : p.cache[1]) +
                                       row0 * p.nkt * (F16 ? 2 : 4);
                    st_stream_cache<W, F16>(crow, (uint32_t)col, ra);
                    st_stream_cache<W, F16>(crow, (uint32_t)(col + d1), rb);
                }
            } else {
                float *const xrow = xsec + (int64_t)(t0 + tt) * ldx;
                st_stream<W>(xrow, (uint32_t)col * 4u, ra);
                st_stream<W>(xrow, (uint32_t)(col + d1) * 4u, rb);
                if (sec > 0 && row >= 0) {
                    void *const crow = static_cast<char *>(cache) + row * p.nkt * (F16 ? 2 : 4);
                    st_stream_cache<W, F16>(crow, (uint32_t)col, ra);
                    st_stream_cache<W, F16>(crow, (uint32_t)(col + d1), rb);
                }
            }
        } else {
            float *xp = xs + (int64_t)(t0 + tt) * ldx;
            st_data<W, false>(xp, ra);
            st_data<W, false>(xp + d1, rb);
            if (sec > 0 && row >= 0) {
                const int64_t off = row * p.nkt + col;
                st_cache<W, F16, false>(cache, off, ra);
                st_cache<W, F16, false>(cache, off + d1, rb);
            }
        }
    }
}

template <int W, bool F16, int TPB, bool STREAM, int NORM, int STYLE, typename TAB>
hipError_t launch_t(const KParams &kp, const TAB &inv, const Plan &pl, hipStream_t st)
{
    const int64_t ntb = pl.grid / pl.ncb;  // token blocks
    const unsigned gy = (unsigned)(ntb < 65535 ? ntb : 65535);
    const unsigned gz = (unsigned)((ntb + gy - 1) / gy);
    hipLaunchKernelGGL((qkv_epilogue_kernel<W, F16, TPB, STREAM, NORM, STYLE, TAB>),
                       dim3((unsigned)pl.ncb, gy, gz), dim3((unsigned)pl.nthr), (unsigned)pl.lds, st,
                       kp, inv);
    return hipGetLastError();
}

// The planner puts one token in each workgroup: the kernel takes any TPB, but
// two or four tokens per workgroup measured slower at every launch size.
template <int W, bool F16, int NORM, int STYLE, typename TAB>
hipError_t launch_s(const KParams &kp, const TAB &inv, const Plan &pl, hipStream_t st)
{
    if (pl.tb != 1)
        return hipErrorInvalidValue;
    return pl.stream ? launch_t<W, F16, 1, true, NORM, STYLE>(kp, inv, pl, st)
                     : launch_t<W, F16, 1, false, NORM, STYLE>(kp, inv, pl, st);
}

template <int W, bool F16, int NORM, typename TAB>
hipError_t launch_n(const KParams &kp, const TAB &inv, const Plan &pl, hipStream_t st)
{
    return pl.style == QKV_ROPE_INTERLEAVED ? launch_s<W, F16, NORM, 1>(kp, inv, pl, st)
                                            : launch_s<W, F16, NORM, 0>(kp, inv, pl, st);
}

template <int W, typename TAB>
hipError_t launch_w(const KParams &kp, const TAB &inv, const Plan &pl, bool f16,
                    hipStream_t st)
{
    const int uph = pl.half / W;
    const bool pow2 = uph <= 64 && (uph & (uph - 1)) == 0;
    if (pl.norm && pow2)
        return f16 ? launch_n<W, true, 2>(kp, inv, pl, st) : launch_n<W, false, 2>(kp, inv, pl, st);
    if (pl.norm)
        return f16 ? launch_n<W, true, 1>(kp, inv, pl, st) : launch_n<W, false, 1>(kp, inv, pl, st);
    return f16 ? launch_n<W, true, 0>(kp, inv, pl, st) : launch_n<W, false, 0>(kp, inv, pl, st);
}

}  // namespace

namespace qkv_detail {

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

const InvTable &handle_inv(qkv_epilogue *h, float theta, int head_dim, float freq_scale)
{
    if (freq_scale == 0.0f)
        freq_scale = 1.0f;
    if (h->inv_hd != head_dim || h->inv_theta != theta || h->inv_scale != freq_scale) {
        host_inv_freq(theta, head_dim, freq_scale, h->inv.v);
        h->inv_hd = head_dim;
        h->inv_theta = theta;
        h->inv_scale = freq_scale;
    }
    return h->inv;
}

// The fused launch behind run_ex (flags 0) and run_qk_norm.
int launch_fused(qkv_epilogue_t *h, const qkv_epilogue_args_t *a, unsigned flags, const float *wq,
                 const float *wk, float eps)
{
    if (!h)
        return QKV_ERR_INVALID_ARG;
    h->msg[0] = 0;
    Plan pl;
    int rc = check_and_plan(a, h->n_ctx, &pl, h->msg, sizeof h->msg, flags, wq, wk, eps);
    if (rc != QKV_OK)
        return rc;
    if (a->nt == 0)
        return QKV_OK;

    const InvTable &inv = handle_inv(h, a->theta, a->head_dim, a->freq_scale);

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
    kp.nt = a->nt;
    kp.hd = a->head_dim;
    kp.half = pl.half;
    kp.uph = pl.half / pl.W;
    kp.qu = a->n_head * kp.uph;
    kp.qku = (a->n_head + a->n_kv_head) * kp.uph;
    kp.vhalf = (int)(pl.nkt / 2);
    kp.U = pl.U;
    kp.cbu = pl.nthr;
    kp.tb = pl.tb;
    kp.uph_mul = ((uint64_t)1 << 40) / (uint64_t)kp.uph + 1;  // ceil: uph never divides 2^40 exactly
    kp.half_mul = ((uint64_t)1 << 40) / (uint64_t)kp.half + 1;
    kp.has_bias = (a->bq ? 1u : 0u) | (a->bk ? 2u : 0u) | (a->bv ? 4u : 0u);
    kp.nw[0] = wq;
    kp.nw[1] = wk;
    kp.eps = (double)eps;

    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    const bool f16 = a->cache_dtype == QKV_CACHE_F16;
    if (pl.half <= kSmallHalf) {
        const InvTableSmall sm = small_table(inv);
        e = pl.W == 4 ? launch_w<4>(kp, sm, pl, f16, st) : launch_w<1>(kp, sm, pl, f16, st);
    } else {
        e = pl.W == 4 ? launch_w<4>(kp, inv, pl, f16, st) : launch_w<1>(kp, inv, pl, f16, st);
    }
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return QKV_OK;
}

}  // namespace qkv_detail

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
    h->inv_theta = 0.0f;
    h->inv_hd = 0;
    h->inv_scale = 0.0f;
    h->msg[0] = 0;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e == hipSuccess)
        e = hipMalloc(reinterpret_cast<void **>(&h->d_err), 16);
    if (e == hipSuccess)
        e = hipMemset(h->d_err, 0, 16);
    // the static workspace's address on this device (the allocation-free
    // projection reports an error if the lookup failed)
    if (e == hipSuccess)
        (void)proj_scratch_setup(h->device);
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
    return launch_fused(h, a, 0u, nullptr, nullptr, 0.0f);
}

int qkv_epilogue_run_qk_norm(qkv_epilogue_t *h, const qkv_epilogue_args_t *a, const float *w_q,
                             const float *w_k, float eps)
{
    return launch_fused(h, a, kPlanBiasOptional | kPlanNorm, w_q, w_k, eps);
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
    // Every launch made before this call, on any stream and from any graph
    // replay, has finished before the word is read.  The device is waited
    // for, not a list of the handle's streams: a caller may have destroyed a
    // stream it launched on since, and graph replays are launches the handle
    // never sees.
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = hipMemcpy(&word, h->d_err, sizeof word, hipMemcpyDeviceToHost);
    // cleared before any later launch can run (the null stream is waited for)
    if (e == hipSuccess && word)
        e = hipMemsetAsync(h->d_err, 0, sizeof word, nullptr);
    if (e == hipSuccess && word)
        e = hipStreamSynchronize(nullptr);
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
    if (g.set(h->device) == hipSuccess) {
        if (h->d_err)
            (void)hipFree(h->d_err);
        if (h->proj_ws)
            (void)hipFree(h->proj_ws);
    }
    delete h;
}

}  // extern "C"
