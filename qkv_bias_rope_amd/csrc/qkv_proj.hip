// qkv_proj.hip -- the concat q|k|v projection with the epilogue in its output
// stage: y = x * W^T (bf16 inputs, f32 accumulation), then bias, NeoX rotary
// embedding, write-back of the q/k/v rows and the K/V cache rows, applied to
// the sums before y is ever written.
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
//  * Tiles of 256 tokens x 256 outputs, four waves of 128 x 128; operands go
//    from HBM straight into a ring of four LDS stages (k sub-tiles of 32,
//    loaded three ahead), XOR-swizzled so fragment reads are conflict-free.
//  * A wave's 128 output columns are one head (hd 128) or two (hd 64), so the
//    NeoX partner of column j (j + hd/2) sits in the same lane, in the MFMA
//    tile hd/64 tiles further on: the rotation needs no data exchange.
//  * 1024+ tokens: the epilogue runs on the accumulators (tiles computed
//    transposed so a lane holds 4 consecutive outputs), with a cos/sin table
//    computed once per launch.  Fewer tokens: the tiles are too few to fill
//    the chip, so k is split across workgroups that store partial tiles to
//    the handle's workspace, and a second kernel sums them in split order and
//    runs the epilogue.
//  * Decode (up to 8 tokens) is a weight-streaming GEMV, not a contraction
//    worth the matrix units: a separate kernel streams W with 16-byte loads,
//    reduces each dot product across the wave and runs the same epilogue.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>

#include "qkv_internal.h"

using namespace qkv_detail;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
    const float *rtab;       // [M][cos half | sin half] (fused long-prompt path)
    int ksplit;              // k splits of the split path
    float *part;             // [ksplit][M][N] partial sums of the split path
    int device;              // the handle's device (launch set-up only)
    bool vec;                // sections, biases, caches 16-byte aligned, strides % 4 == 0
};

// cache row of token t (slot * n_ctx + pos), or -1 when pos or slot is out
// of range (the caller then sets the error word)
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
// cos/sin table of a launch: row t holds cos then sin of pos[t] * inv[i],
// i < half (f32 angle; sin/cos in double rounded to f32).  Every column
// block reads it instead of recomputing it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_table_kernel(const int32_t *pos, int M, int half,
                                                         InvTable inv, float *tab)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * half)
        return;
    const int t = (int)(idx / half), i = (int)(idx - (int64_t)t * half);
    const float ang = (float)pos[t] * inv.v[i];
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    tab[(int64_t)t * 2 * half + i] = (float)cd;
    tab[(int64_t)t * 2 * half + half + i] = (float)sd;
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles, operands loaded straight into LDS
// ---------------------------------------------------------------------------
// Eight waves, two per SIMD: wave (wm, wn) owns 128 tokens (wm) x 64 outputs,
// the two 32-column MFMA tiles f0 and f0 + hd/64 of one head, so the NeoX
// partner of every output sits in the same lane and register of the other
// tile.  128 accumulators per lane leave room for two waves per SIMD, which
// is what keeps the LDS busy: on gfx950 conflict-free 16-byte LDS reads
// reach ~135 B/clk per CU with one wave per SIMD and ~225 with two.
//
// k advances in sub-tiles of 32 through a ring of four LDS stages (32 KB
// each: 256 token rows of A and 256 weight rows of B, 64 bytes per row),
// filled by global->LDS loads (64 lanes x 16 bytes per instruction) issued
// three sub-tiles ahead.  Chunk c of row r sits in slot c ^ g(r),
// g(r) = ((r >> 1) ^ (r >> 3)) & 3: the 16-byte fragment reads of 16
// consecutive rows hit distinct banks.
//
// Per sub-tile s (two k steps of 16, 8 products each):
//   products of step 0 (first half); read step-1 fragments; products of
//   step 0 (second half); products of step 1 (first half); wait for this
//   wave's loads of sub-tile s+1 and meet the other waves (after which stage
//   s is free and sub-tile s+1 is visible); load sub-tile s+4 into stage s;
//   read step-0 fragments of sub-tile s+1; products of step 1 (second half).
namespace big {
constexpr int BN = 256, BK = 32, NSTAGE = 4;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRow = BK * 2;                  // 64 bytes
constexpr int kRegionB = BN * kRow;           // 16 KB of weight rows per stage
constexpr int kInstB = BN / 16 / kWaves;      // weight-row loads per wave and sub-tile (2)

// the tile shape for MI token tiles of 32 per wave (two waves along tokens)
template <int MI>
struct Shape {
    static constexpr int BM = 2 * MI * 32;                       // 64, 128 or 256 tokens
    static constexpr int kRegionA = BM * kRow;
    static constexpr int kStage = kRegionA + kRegionB;
    static constexpr int kLds = NSTAGE * kStage;                 // 80, 96 or 128 KB
    // token-row loads per wave and sub-tile: BM/16 instructions over 8 waves,
    // at least one (with BM = 64 waves 4-7 repeat the loads of waves 0-3,
    // same rows into the same slots)
    static constexpr int kInstA = BM / 16 >= kWaves ? BM / 16 / kWaves : 1;
    static constexpr int kLoads = kInstA + kInstB;
};

// s_waitcnt immediate that waits for vmcnt <= v only
constexpr int vmcnt_wait(int v)
{
    return (v & 15) | ((v >> 4) << 14) | (0xF << 8) | (7 << 4);
}

__device__ __forceinline__ int swz(int r)
{
    return ((r >> 1) ^ (r >> 3)) & 3;
}
}  // namespace big

// MODE 0: the fused output stage below (one k range per tile).  MODE 1: k is
// split p.ksplit ways across workgroups and each stores its partial y tile to
// p.part; proj_split_epilogue_kernel sums the partials and finishes.  MI:
// token tiles of 32 per wave (4 for long prompts; 2 or 1 for small batches,
// whose tokens would otherwise mostly be padding).
template <bool F16, int HD, int MODE, int MI>
__global__ __launch_bounds__(big::kThreads) void proj_mfma_big_kernel(ProjParams p, InvTable inv)
{
    using namespace big;
    using S = Shape<MI>;
    constexpr int BM = S::BM;
    extern __shared__ __align__(16) unsigned char lds[];
    constexpr int HALF = HD / 2;
    constexpr int PT = HALF / 32;                 // tile distance of NeoX partners

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    // the wave's two output tiles (of the block's 8): f0 and f0 + PT
    const int f0 = (wn / PT) * (2 * PT) + wn % PT;
    const int nblk = p.N / BN + (p.N % BN ? 1 : 0);
    const int mblk = (p.M + BM - 1) / BM;
    const int tile = (int)blockIdx.x % (nblk * mblk);
    const int split = (int)blockIdx.x / (nblk * mblk);
    const int n0 = (tile % nblk) * BN;
    const int m0 = (tile / nblk) * BM;

    // loads: each instruction moves 16 rows (64 lanes x 16 bytes); token-row
    // instruction j of wave w covers rows ra = 16 (w kInstA + j) mod BM (+ lane/4),
    // weight-row instruction j rows rb = 16 (w kInstB + j); lane%4 is the LDS
    // slot and the chunk it holds is slot ^ g(row).  Offsets are bytes from
    // x / w (both < 2 GiB).
    const int lrow = lane >> 2, slot = lane & 3;
    // (fixed-size arrays: with a size that depends on MI, captured by the
    // lambda below, hipcc's host pass silently emitted no launch stub)
    static_assert(S::kInstA <= 2, "token-row loads per wave");
    uint32_t aoff[2], boff[kInstB];
    int arow0[2], brow0[kInstB];
#pragma unroll
    for (int j = 0; j < S::kInstA; ++j) {
        arow0[j] = (16 * (wave * S::kInstA + j)) % BM;
        const int r = arow0[j] + lrow;
        const int chunk = slot ^ big::swz(r);
        aoff[j] = (uint32_t)((int64_t)min(m0 + r, p.M - 1) * p.ld_x * 2) + chunk * 16;
    }
#pragma unroll
    for (int j = 0; j < kInstB; ++j) {
        brow0[j] = 16 * (wave * kInstB + j);
        const int r = brow0[j] + lrow;
        const int chunk = slot ^ big::swz(r);
        boff[j] = (uint32_t)((int64_t)min(n0 + r, p.N - 1) * p.K * 2) + chunk * 16;
    }
    const unsigned char *xb = reinterpret_cast<const unsigned char *>(p.x);
    const unsigned char *wb = reinterpret_cast<const unsigned char *>(p.w);
    typedef __attribute__((address_space(3))) void lds_t;
    // this workgroup's sub-tiles [kt0, kt0 + KT) of the k range
    const int KT_all = p.K / BK;
    const int kt0 = (int)((int64_t)split * KT_all / p.ksplit);
    const int KT = (int)((int64_t)(split + 1) * KT_all / p.ksplit) - kt0;
    // local sub-tile st (clamped to the last one: the loop stays uniform)
    auto issue = [&](int st) {
        const int stage = st % NSTAGE;
        const uint32_t kb = (uint32_t)(kt0 + min(st, KT - 1)) * (BK * 2);
        unsigned char *sa = lds + stage * S::kStage;
        unsigned char *sb = sa + S::kRegionA;
#pragma unroll
        for (int j = 0; j < S::kInstA; ++j)
            __builtin_amdgcn_global_load_lds(xb + aoff[j] + kb, (lds_t *)(sa + arow0[j] * kRow), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < kInstB; ++j)
            __builtin_amdgcn_global_load_lds(wb + boff[j] + kb, (lds_t *)(sb + brow0[j] * kRow), 16, 0, 0);
    };

    // acc[f * MI + ti]: output tile f (0, 1) x token tile ti
    f32x16 acc[2 * MI];
#pragma unroll
    for (int q = 0; q < 2 * MI; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[q][v] = 0.0f;

    // fragment reads: lane reads row lr of each 32-row tile, chunk 2*ks + hi
    const int lr = lane & 31, hi = lane >> 5;
    const int g = big::swz(lr);                 // tiles start at multiples of 32
    const int abase = (wm * MI * 32 + lr) * kRow;
    const int bbase0 = S::kRegionA + (f0 * 32 + lr) * kRow;
    const int bbase1 = bbase0 + PT * 32 * kRow;
    const int k0off = ((0 + hi) ^ g) * 16;      // step 0: chunk hi
    const int k1off = ((2 + hi) ^ g) * 16;      // step 1: chunk 2 + hi

    bf16x8 a0[MI], b0[2], a1[MI], b1[2];
    auto read_frags = [&](const unsigned char *s, int koff, bf16x8 (&fa)[MI], bf16x8 (&fb)[2]) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            fa[mi] = *reinterpret_cast<const bf16x8 *>(s + abase + mi * 32 * kRow + koff);
        fb[0] = *reinterpret_cast<const bf16x8 *>(s + bbase0 + koff);
        fb[1] = *reinterpret_cast<const bf16x8 *>(s + bbase1 + koff);
    };
    // MODE 0 computes each tile transposed (32 outputs x 32 tokens, the
    // weight fragment as the A operand), so a lane ends up holding 4
    // consecutive outputs of a token; MODE 1 keeps tokens x outputs, so one
    // store instruction covers 32 consecutive outputs of a row
    // half h takes products q = f*MI + ti in [h*MI, (h+1)*MI)
    auto mfma_half = [&](int h, const bf16x8 (&fa)[MI], const bf16x8 (&fb)[2]) {
#pragma unroll
        for (int q = h * MI; q < (h + 1) * MI; ++q) {
            const int f = q / MI, ti = q % MI;
            if constexpr (MODE == 0)
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[f], fa[ti], acc[q], 0, 0, 0);
            else
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ti], fb[f], acc[q], 0, 0, 0);
        }
    };

    // prologue: sub-tiles 0..3 in flight, sub-tile 0 landed everywhere:
    // vmcnt <= 3 * loads per sub-tile; no lgkm/exp wait
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st)
        issue(st);
    constexpr int kWaitFirst = vmcnt_wait(3 * S::kLoads);
    constexpr int kWaitNext = vmcnt_wait(2 * S::kLoads);
    __builtin_amdgcn_s_waitcnt(kWaitFirst);
    __syncthreads();
    read_frags(lds, k0off, a0, b0);

    for (int kt = 0; kt < KT; ++kt) {
        const unsigned char *s = lds + (kt % NSTAGE) * S::kStage;
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(s, k1off, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(1, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(0, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        // this wave's loads of sub-tile kt+1 have landed once at most the two
        // later groups (kt+2, kt+3) are outstanding
        __builtin_amdgcn_s_waitcnt(kWaitNext);
        __syncthreads();
        issue(kt + NSTAGE);
        read_frags(lds + ((kt + 1) % NSTAGE) * S::kStage, k0off, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(1, a1, b1);
    }
    // the clamped reloads of the last iterations must land before the wave
    // leaves (they write this block's LDS)
    __builtin_amdgcn_s_waitcnt(0);

    const int col0 = n0 + f0 * 32;                 // first output column of tile f = 0
    if (col0 >= p.N)
        return;
    if constexpr (MODE == 1) {
        // partial y of this split: lane (lr, hi) holds output f*PT*32 + lr
        // (from col0) of tokens ti*32 + 8(v/4) + 4hi + v%4
        float *const out = p.part + (int64_t)split * p.M * p.N + col0 + lr;
#pragma unroll
        for (int ti = 0; ti < MI; ++ti)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = m0 + wm * MI * 32 + ti * 32 + 8 * (v / 4) + 4 * hi + (v & 3);
                if (t >= p.M)
                    continue;
                float *const o = out + (int64_t)t * p.N;
                o[0] = acc[ti][v];
                o[PT * 32] = acc[MI + ti][v];
            }
        return;
    }

    // ---- epilogue ---------------------------------------------------------
    // Lane (lr, hi) holds, for token ti*32 + lr of the wave's 128, the
    // outputs col0 + f*HALF + 8g + 4hi + e (e < 4) in acc[f*MI + ti][4g + e]:
    // four consecutive columns, stored with one 16-byte (f32) or 8-byte
    // (f16) store; f = 1 is the NeoX partner of f = 0.  cos/sin come from the
    // launch's table (16-byte reads).
    const int sec = col0 < p.nqt ? 0 : (col0 < p.nqt + p.nkt ? 1 : 2);
    const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
    float *const out = p.out[sec];
    const int64_t ldo = p.ld[sec];
    const float *const bias = p.b[sec];
    void *const cache = sec == 1 ? p.cache[0] : p.cache[1];
    const int cs = col0 - sbase + 4 * hi;          // section column of (f = 0, g = 0)
    const int ih = (f0 * 32) % HD;                 // pair index of the tile's first column

    // this lane's 32 bias values, loaded once
    const FVec<4> zero = {{0.f, 0.f, 0.f, 0.f}};
    FVec<4> bias0[4], bias1[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        bias0[g] = bias ? ld_vec<4>(bias + cs + 8 * g) : zero;
        bias1[g] = bias ? ld_vec<4>(bias + cs + 8 * g + HALF) : zero;
    }

#pragma unroll
    for (int ti = 0; ti < MI; ++ti) {
        const int t = m0 + wm * MI * 32 + ti * 32 + lr;
        if (t >= p.M)
            continue;
        const int64_t row = sec > 0 ? cache_row(p, t) : -1;
        float *const orow = out + (int64_t)t * ldo;
        // all of this token's cos/sin values first: one wait per token
        const float *const trow = p.rtab + (int64_t)t * 2 * HALF + ih + 4 * hi;
        FVec<4> cv[4], sv[4];
        if (sec < 2) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                cv[g] = ld_vec<4>(trow + 8 * g);
                sv[g] = ld_vec<4>(trow + HALF + 8 * g);
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c0 = cs + 8 * g, c1 = c0 + HALF;
            FVec<4> y0, y1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y0.e[e] = acc[ti][4 * g + e] + bias0[g].e[e];
                y1.e[e] = acc[MI + ti][4 * g + e] + bias1[g].e[e];
            }
            if (sec < 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rot(y0.e[e], y1.e[e], cv[g].e[e], sv[g].e[e]);
            }
            st_data<4, false>(orow + c0, y0);
            st_data<4, false>(orow + c1, y1);
            if (row >= 0) {
                st_cache<4, F16, false>(cache, row * p.nkt + c0, y0);
                st_cache<4, F16, false>(cache, row * p.nkt + c1, y1);
            }
        }
        if (sec > 0 && row < 0 && hi == 0)
            atomicOr(p.err, 1u);
    }
}

// ---------------------------------------------------------------------------
// split path, second step: y = sum of the k-split partials (in split order,
// so the result does not depend on timing), then the epilogue.  One thread
// per column pair (j, j + hd/2) of a head (the v section pairs its columns
// the same way, without the rotation); cos/sin from the launch's table.
// ---------------------------------------------------------------------------
template <bool F16, int HD>
__global__ __launch_bounds__(256) void proj_split_epilogue_kernel(ProjParams p)
{
    constexpr int HALF = HD / 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int pairs = p.N / 2;
    if (idx >= (int64_t)p.M * pairs)
        return;
    const int t = (int)(idx / pairs);
    const int pr = (int)(idx - (int64_t)t * pairs);
    const int head = pr / HALF, i = pr - head * HALF;
    const int c0 = head * HD + i, c1 = c0 + HALF;
    const float *src = p.part + (int64_t)t * p.N;
    float y0 = src[c0], y1 = src[c1];
    for (int sp = 1; sp < p.ksplit; ++sp) {
        src += (int64_t)p.M * p.N;
        y0 = y0 + src[c0];
        y1 = y1 + src[c1];
    }
    const int sec = c0 < p.nqt ? 0 : (c0 < p.nqt + p.nkt ? 1 : 2);
    const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
    const int s0 = c0 - sbase, s1 = c1 - sbase;
    const float *bias = p.b[sec];
    if (bias) {
        y0 = y0 + bias[s0];
        y1 = y1 + bias[s1];
    }
    if (sec < 2) {
        const float *trow = p.rtab + (int64_t)t * HD;
        rot(y0, y1, trow[i], trow[HALF + i]);
    }
    float *out = p.out[sec] + (int64_t)t * p.ld[sec];
    out[s0] = y0;
    out[s1] = y1;
    if (sec > 0) {
        const int64_t row = cache_row(p, t);
        void *cache = sec == 1 ? p.cache[0] : p.cache[1];
        if (row >= 0) {
            put_cache<F16>(cache, row * p.nkt + s0, y0);
            put_cache<F16>(cache, row * p.nkt + s1, y1);
        } else if (pr == p.nqt / 2) {   // the first k pair reports the token
            atomicOr(p.err, 1u);
        }
    }
}

// ---------------------------------------------------------------------------
// decode (1-8 tokens): weight-streaming GEMV + epilogue
// ---------------------------------------------------------------------------
// One wave per NeoX pair of weight rows (j and j + hd/2 of a head; in the v
// section the same pairing just groups rows), four waves per block.  Lane l
// takes the 16-byte chunks l, l+64, ... of both rows, U chunks in flight
// per row, and keeps NT running sums per row (v_dot2_f32_bf16: two bf16
// products into the f32 sum per instruction); a butterfly over the wave
// completes the dot products, and lane t < nt finishes token t: bias, the
// rotation of the pair, write-back and the cache store.
constexpr int kGemvTok = 8;          // the GEMV path takes up to 8 tokens
constexpr int kGemvWaves = 4;

// U: 16-byte chunks of each row in flight per lane and step; the launcher
// picks U dividing the chunks per lane (hidden/512) when it can, since a
// partial last step costs as much as a full one.  P: NeoX pairs per wave (4
// for 5-8 tokens, so each x chunk loaded serves eight weight rows).
template <bool F16, int HD, int NT, int U, int P>
__global__ __launch_bounds__(64 * kGemvWaves) void proj_gemv_kernel(ProjParams p, InvTable inv)
{
    constexpr int HALF = HD / 2;
    constexpr int R = 2 * P;                 // weight rows per wave
    const int lane = (int)threadIdx.x & 63;
    const int pair0 = ((int)blockIdx.x * kGemvWaves + ((int)threadIdx.x >> 6)) * P;
    if (pair0 >= p.N / 2)
        return;
    const int nchunk = p.K / 8;
    // rows 2q and 2q+1 are columns c0 and c0 + hd/2 of pair pair0 + q
    const uint16_t *wr[R];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int pr = pair0 + q;
        const int c0 = (pr / HALF) * HD + pr % HALF;
        wr[2 * q] = p.w + (int64_t)c0 * p.K;
        wr[2 * q + 1] = p.w + (int64_t)(c0 + HALF) * p.K;
    }
    const uint16_t *xr[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        xr[t] = p.x + (int64_t)min(t, p.M - 1) * p.ld_x;

    float d[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            d[r][t] = 0.0f;
    for (int cb = lane; cb < nchunk; cb += 64 * U) {
        u32x4 wv[U][R], xv[U][NT];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + 64 * u;
            ok[u] = c < nchunk;
            const int cc = ok[u] ? c : 0;    // past the row end: reload chunk 0, weight 0
            // the weights are read once per call: nontemporal
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[r] + cc * 8));
#pragma unroll
            for (int t = 0; t < NT; ++t)
                xv[u][t] = *reinterpret_cast<const u32x4 *>(xr[t] + cc * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // each dword holds two consecutive bf16 of a row (x and W alike):
            // one dot2 adds both exact products to the f32 sum.  The pairs are
            // taken from the whole 16-byte vector by shuffles: bit-casting
            // single dwords of it compiled to one-dword loads reused for all
            // four pairs (checked in the ISA).
            bf16x8 xx8[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                xx8[t] = __builtin_bit_cast(bf16x8, xv[u][t]);
#define QKV_PAIR(v8, e) __builtin_shufflevector(v8, v8, 2 * (e), 2 * (e) + 1)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bf16x8 w8 = __builtin_bit_cast(
                    bf16x8, ok[u] ? wv[u][r] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t], 0), QKV_PAIR(w8, 0), d[r][t], false);
                    d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t], 1), QKV_PAIR(w8, 1), d[r][t], false);
                    d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t], 2), QKV_PAIR(w8, 2), d[r][t], false);
                    d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t], 3), QKV_PAIR(w8, 3), d[r][t], false);
                }
            }
#undef QKV_PAIR
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1)
                d[r][t] += __shfl_xor(d[r][t], m, 64);

    if (lane >= NT || lane >= p.M)
        return;
    const int t = lane;
#pragma unroll
    for (int q = 0; q < P; ++q) {
        float y0 = d[2 * q][0], y1 = d[2 * q + 1][0];
#pragma unroll
        for (int u = 1; u < NT; ++u)
            if (t == u) {
                y0 = d[2 * q][u];
                y1 = d[2 * q + 1][u];
            }
        const int pr = pair0 + q;
        const int i = pr % HALF;
        const int c0 = (pr / HALF) * HD + i;     // global output column of the pair's first row
        const int sec = c0 < p.nqt ? 0 : (c0 < p.nqt + p.nkt ? 1 : 2);
        const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
        const int s0 = c0 - sbase, s1 = s0 + HALF;   // columns inside the section
        const float *bias = p.b[sec];
        if (bias) {
            y0 = y0 + bias[s0];
            y1 = y1 + bias[s1];
        }
        if (sec < 2) {
            const float ang = (float)p.pos[t] * inv.v[i];
            double sd, cd;
            sincos((double)ang, &sd, &cd);
            rot(y0, y1, (float)cd, (float)sd);
        }
        float *out = p.out[sec];
        out[(int64_t)t * p.ld[sec] + s0] = y0;
        out[(int64_t)t * p.ld[sec] + s1] = y1;
        if (sec > 0) {
            const int64_t row = cache_row(p, t);
            void *cache = sec == 1 ? p.cache[0] : p.cache[1];
            if (row >= 0) {
                put_cache<F16>(cache, row * p.nkt + s0, y0);
                put_cache<F16>(cache, row * p.nkt + s1, y1);
            } else if (i == 0) {
                atomicOr(p.err, 1u);
            }
        }
    }
}

// Launch choice.  Decode (1-8 tokens): the GEMV.  Long prompts (1024+ tokens,
// 16-byte aligned sections): the cos/sin table and the fused 256 x 256 kernel.
// Otherwise (a batch of a few hundred tokens has too few 256 x 256 tiles to
// fill the chip, e.g. 28 at the 14B shape): the table, the 256 x 256 kernel
// with k split so the launch has about one workgroup per CU, each split
// storing its partial tile, and a summing epilogue kernel.
constexpr int kLargeM = 1024;
constexpr int kTargetGroups = 256;

// Raise the kernel's dynamic-LDS limit to what it uses (up to 128 KB), once
// per kernel and device (the caller has made the handle's device current).
template <bool F16, int HD, int MODE, int MI>
hipError_t set_big_lds(int device)
{
    static std::atomic<unsigned long long> done{0};
    const unsigned long long bit = 1ull << (device & 63);
    if (done.load(std::memory_order_acquire) & bit)
        return hipSuccess;
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&proj_mfma_big_kernel<F16, HD, MODE, MI>),
        hipFuncAttributeMaxDynamicSharedMemorySize, big::Shape<MI>::kLds);
    if (e == hipSuccess && device < 64)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

// token tiles per wave of the split path: the smallest tile height that
// holds the batch (64, 128, then 256 tokens)
int split_mi(int M)
{
    return M <= 64 ? 1 : (M <= 128 ? 2 : 4);
}

// the number of k splits of the split path for this shape
int choose_ksplit(int M, int N, int K)
{
    const int bm = 64 * split_mi(M);
    const int tiles = ((N + big::BN - 1) / big::BN) * ((M + bm - 1) / bm);
    int s = (kTargetGroups + tiles / 2) / tiles;
    const int max_s = K / big::BK / 4;   // at least 4 sub-tiles per split
    if (s > max_s)
        s = max_s;
    return s < 1 ? 1 : s;
}

// chunks per row and step of the GEMV: the largest of 8..4 dividing the
// chunks per lane, else the one wasting the fewest slots
int gemv_step(int K)
{
    const int c = (K / 8 + 63) / 64;   // 16-byte chunks per lane and row
    int best = 4, waste = 1 << 30;
    for (int u = 8; u >= 4; --u) {
        const int w = (c + u - 1) / u * u - c;
        if (w < waste) {
            best = u;
            waste = w;
        }
    }
    return best;
}

template <bool F16, int HD, int NT>
hipError_t launch_gemv(const ProjParams &pp, const InvTable &inv, hipStream_t st, int u)
{
    const int blocks = (pp.N / 2 + kGemvWaves - 1) / kGemvWaves;
    const dim3 grid(blocks), block(64 * kGemvWaves);
    switch (u) {
    case 8: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 8, 1>), grid, block, 0, st, pp, inv); break;
    case 7: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 7, 1>), grid, block, 0, st, pp, inv); break;
    case 6: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 6, 1>), grid, block, 0, st, pp, inv); break;
    case 5: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 5, 1>), grid, block, 0, st, pp, inv); break;
    default: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 4, 1>), grid, block, 0, st, pp, inv); break;
    }
    return hipGetLastError();
}

// 5-8 tokens: four pairs per wave, one chunk per row in flight (each x
// chunk loaded serves eight weight rows; measured 24.5 us at 14B against
// 27.9 with two pairs and 32 on the MFMA split path)
template <bool F16, int HD>
hipError_t launch_gemv8(const ProjParams &pp, const InvTable &inv, hipStream_t st)
{
    const int blocks = (pp.N / 8 + kGemvWaves - 1) / kGemvWaves;
    hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, 8, 1, 4>), dim3(blocks), dim3(64 * kGemvWaves), 0,
                       st, pp, inv);
    return hipGetLastError();
}

template <bool F16, int HD, int MI>
hipError_t launch_split_gemm(const ProjParams &pp, const InvTable &inv, hipStream_t st, int nblk)
{
    using S = big::Shape<MI>;
    hipError_t e = set_big_lds<F16, HD, 1, MI>(pp.device);
    if (e != hipSuccess)
        return e;
    const int mblk = (pp.M + S::BM - 1) / S::BM;
    hipLaunchKernelGGL((proj_mfma_big_kernel<F16, HD, 1, MI>), dim3(nblk * mblk * pp.ksplit),
                       dim3(big::kThreads), (unsigned)S::kLds, st, pp, inv);
    return hipGetLastError();
}

template <bool F16, int HD>
hipError_t launch_proj(const ProjParams &pp, const InvTable &inv, hipStream_t st)
{
    if (pp.M <= kGemvTok) {
        const int u = gemv_step(pp.K);
        if (pp.M == 1)
            return launch_gemv<F16, HD, 1>(pp, inv, st, u);
        if (pp.M == 2)
            return launch_gemv<F16, HD, 2>(pp, inv, st, u);
        if (pp.M <= 4)
            return launch_gemv<F16, HD, 4>(pp, inv, st, u);
        return launch_gemv8<F16, HD>(pp, inv, st);
    }
    const int nblk = pp.N / big::BN + (pp.N % big::BN ? 1 : 0);
    const int64_t n_tab = (int64_t)pp.M * (HD / 2);
    if (pp.M >= kLargeM && pp.vec) {
        using S = big::Shape<4>;
        hipError_t e = set_big_lds<F16, HD, 0, 4>(pp.device);
        if (e != hipSuccess)
            return e;
        const int mblk = (pp.M + S::BM - 1) / S::BM;
        hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0,
                           st, pp.pos, pp.M, HD / 2, inv, const_cast<float *>(pp.rtab));
        hipLaunchKernelGGL((proj_mfma_big_kernel<F16, HD, 0, 4>), dim3(nblk * mblk),
                           dim3(big::kThreads), (unsigned)S::kLds, st, pp, inv);
        return hipGetLastError();
    }
    // split path: the table, the GEMM writing k-split partials, the summing epilogue
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0, st,
                       pp.pos, pp.M, HD / 2, inv, const_cast<float *>(pp.rtab));
    const int mi = split_mi(pp.M);
    hipError_t e = mi == 1 ? launch_split_gemm<F16, HD, 1>(pp, inv, st, nblk)
                 : mi == 2 ? launch_split_gemm<F16, HD, 2>(pp, inv, st, nblk)
                           : launch_split_gemm<F16, HD, 4>(pp, inv, st, nblk);
    if (e != hipSuccess)
        return e;
    const int64_t n_pairs = (int64_t)pp.M * (pp.N / 2);
    hipLaunchKernelGGL((proj_split_epilogue_kernel<F16, HD>), dim3((unsigned)((n_pairs + 255) / 256)),
                       dim3(256), 0, st, pp);
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
    if (pa->hidden <= 0 || pa->hidden % 64 != 0)
        return fail(h, QKV_ERR_INVALID_ARG, "hidden must be a positive multiple of 64, got %d",
                    pa->hidden);
    if (pl.nqt % 128 != 0 || pl.nkt % 128 != 0)
        return fail(h, QKV_ERR_UNSUPPORTED,
                    "the projection path needs q and k/v widths that are multiples of 128 "
                    "(got %lld and %lld)",
                    (long long)pl.nqt, (long long)pl.nkt);
    if (N > INT32_MAX / 2)
        return fail(h, QKV_ERR_INVALID_ARG, "q|k|v width too large");
    // the kernels address x and w with 32-bit byte offsets
    if ((int64_t)a->nt * (pa->ld_x ? pa->ld_x : pa->hidden) * 2 > INT32_MAX ||
        N * pa->hidden * 2 > INT32_MAX)
        return fail(h, QKV_ERR_INVALID_ARG, "x and w must each span less than 2 GiB");
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
    pp.vec = pl.W == 4;
    pp.rtab = nullptr;
    pp.ksplit = 1;
    pp.part = nullptr;
    pp.device = h->device;

    const InvTable &inv = handle_inv(h, a->theta, a->head_dim, a->freq_scale);
    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    if (pp.M > kGemvTok) {
        // the MFMA paths read a [nt][head_dim] f32 cos/sin table from the
        // handle's workspace, and the split path also keeps its [splits][nt][N]
        // partial sums there; a larger request than any before grows it
        // (after the device has finished with the old one)
        const bool fused = pp.M >= kLargeM && pp.vec;
        pp.ksplit = fused ? 1 : choose_ksplit(pp.M, pp.N, pp.K);
        const size_t tab = (size_t)pp.M * (size_t)a->head_dim * sizeof(float);
        const size_t need = tab + (fused ? 0 : (size_t)pp.ksplit * pp.M * pp.N * sizeof(float));
        if (h->proj_ws_bytes < need) {
            e = hipDeviceSynchronize();
            if (e == hipSuccess && h->proj_ws)
                e = hipFree(h->proj_ws);
            h->proj_ws = nullptr;
            h->proj_ws_bytes = 0;
            if (e == hipSuccess)
                e = hipMalloc(&h->proj_ws, need);
            if (e != hipSuccess) {
                h->proj_ws = nullptr;
                return fail(h, QKV_ERR_HIP, "workspace of %zu bytes: %s", need,
                            hipGetErrorString(e));
            }
            h->proj_ws_bytes = need;
        }
        pp.rtab = static_cast<const float *>(h->proj_ws);
        pp.part = reinterpret_cast<float *>(static_cast<char *>(h->proj_ws) + tab);
    }
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
