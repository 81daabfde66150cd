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
//  * Eight-wave tiles of 256 x 256, 256 x 128, 128 x 128 or 64 x 256 tokens x
//    outputs, picked per launch by a cost model; operands go from HBM
//    straight into a ring of LDS stages 64 deep in k (two to four of them,
//    as many as fit), XOR-swizzled so fragment reads are conflict-free.
//  * A wave's 64 output columns are the j and j + hd/2 halves of a head's
//    NeoX pairs, so the partner of every output sits in the same lane, in the
//    other MFMA tile: the rotation needs no data exchange.
//  * When the tiles fill the chip the epilogue runs on the accumulators
//    (tiles computed transposed so a lane holds 4 consecutive outputs), with
//    cos/sin and cache rows tabled once per launch.  With too few tiles k is
//    split across workgroups that store partial tiles to the handle's
//    workspace, and a second kernel sums them in split order and runs the
//    epilogue.
//  * Decode (up to 4 tokens) is a weight-streaming GEMV, not a contraction
//    worth the matrix units: a separate kernel streams W with 16-byte loads,
//    reduces each dot product across the wave and runs the same epilogue.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
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
    const uint16_t *wsec[3]; // weight rows of the q, k, v sections ([nqt|nkt|nkt][K]): bf16, or
                             // E4M3 bytes when w8
    bool sep;                // the sections are three matrices (else rows of one concat matrix)
    bool w8;                 // E4M3 weights with one f32 scale per output row
    const float *wscale;     // [N] row scales (w8)
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
    const float *rtab;       // [M][cos half | sin half] of the launch (MFMA path)
    const int64_t *rows;     // [M] cache row of each token, or -1 (MFMA path)
    int ksplit;              // k splits of the MFMA path
    float *part;             // [ksplit][M][N] partial sums when ksplit > 1
    int device;              // the handle's device (launch set-up only)
    int style;               // QKV_ROPE_NEOX (pair j, j + hd/2) or QKV_ROPE_INTERLEAVED (2i, 2i + 1)
    bool vec;                // sections, biases, caches 16-byte aligned, strides % 4 == 0
};

// weight row of output n: row n - section base of its section's matrix (SEP:
// three matrices), or row n of the concat matrix; rows of K weights of 2
// bytes (bf16) or 1 byte (W8: E4M3)
template <bool SEP, bool W8>
__device__ __forceinline__ const unsigned char *weight_row(const ProjParams &p, int n)
{
    constexpr int64_t kEl = W8 ? 1 : 2;
    int s = 0, base = 0;
    if (SEP && n >= p.nqt + p.nkt) {
        s = 2;
        base = p.nqt + p.nkt;
    } else if (SEP && n >= p.nqt) {
        s = 1;
        base = p.nqt;
    }
    return reinterpret_cast<const unsigned char *>(p.wsec[s]) + (int64_t)(n - base) * p.K * kEl;
}

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
// Per-launch tables of the MFMA path: row t of tab holds cos then sin of
// pos[t] * inv[i], i < half (f32 angle; sin/cos in double rounded to f32), and
// rows[t] is token t's cache row (slot * n_ctx + pos, or -1 when out of
// range).  Every column block reads them instead of recomputing them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_table_kernel(ProjParams p, InvTableSmall inv, float *tab,
                                                         int64_t *rows)
{
    const int half = p.half;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * half)
        return;
    const int t = (int)(idx / half), i = (int)(idx - (int64_t)t * half);
    const float ang = (float)p.pos[t] * inv.v[i];
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    tab[(int64_t)t * 2 * half + i] = (float)cd;
    tab[(int64_t)t * 2 * half + half + i] = (float)sd;
    if (i == 0)
        rows[t] = cache_row(p, t);
}

// ---------------------------------------------------------------------------
// The MFMA path (9+ tokens): eight-wave tiles, operands loaded straight into
// LDS, the epilogue on the accumulators
// ---------------------------------------------------------------------------
// A workgroup computes a BM x BN tile of y with eight waves.  Wave (wm, wn)
// owns MI*32 tokens x 64 outputs: the two 32-column MFMA tiles of one NeoX
// pair group, i.e. columns j and j + hd/2 of a head (for hd 128 the tiles lo
// and lo + 2, for hd 64 lo and lo + 1), so the rotation partner of every
// output sits in the same lane and register of the other tile.  WN waves
// along the outputs (BN = 64 WN), 8/WN along the tokens (BM = 8/WN * MI * 32),
// so one kernel serves long prompts (256 x 256) and batches whose tokens
// would mostly be padding in a tall tile (64 x 256, 256 x 64, ...).  Each
// 32 x 32 tile is computed transposed (the weight fragment as the A operand),
// so a lane holds 4 consecutive outputs of one token: 16-byte stores.
//
// k advances in stages of BK = 64 (BM token rows of A and BN weight rows of
// B, 128 bytes per row) through a ring of NSTAGE LDS stages -- as many as the
// 160 KB hold, at most 4: 2 for 256 x 256, 3 for 256 x 128, 4 for the small
// tiles -- filled by global->LDS loads (64 lanes x 16 bytes per instruction)
// issued NSTAGE - 1 stages ahead.  On MI355X 64-deep stages ran 5-20%
// faster than 32-deep ones (two k steps per barrier) and 128-deep ones were
// slower again: a deeper stage amortises the barrier and the ring's refill
// latency, until the ring gets too shallow to hide HBM.  Chunk c of row r sits in
// slot c ^ g(r), with g(r) = (r >> 1) & 7 for 128-byte rows ((r >> 2) & 3
// for 64-byte rows, r & 15 for 256-byte rows), which makes the 16-byte
// fragment reads (16 rows of a quarter wave, one chunk each) conflict-free
// on gfx950: a probe under rocprofv3 reads 4 LDS cycles per ds_read_b128,
// where the swizzle ((r >> 1) ^ (r >> 3)) & 3 -- conflict-free on paper for
// 64 four-byte banks serving 16 lanes at a time -- takes 8.  The fragments
// of a stage's k steps are double-buffered in registers; per pair of steps
// j, j + 1:
//   products of step j, with the step-(j+1) fragment reads spread among
//   them (one read after each MFMA); products of step j+1, with the
//   step-(j+2) reads spread among them -- or, after the stage's last step:
//   its first half; wait for this wave's loads of the next stage and meet
//   the other waves (after which this stage is free and the next visible),
//   refill this stage NSTAGE ahead and read the next stage's first
//   fragments; its second half.  Bunched after a step's first half
//   instead, the reads have four MFMAs in front of their first use, and the
//   4096-token launch measured 1-2% (bf16) and 1-4% (E4M3) slower.
//
// The grid is tiles x S: with S = 1 each workgroup finishes its tile (the
// epilogue below); when the tiles are too few to fill the chip, k is split S
// ways, each split stores its partial tile ([S][M][N] in the workspace) and
// proj_split_epilogue_kernel sums the partials in split order (the same
// additions every run) and finishes.  Consecutive blocks take consecutive
// tiles of the same k range, so the tiles in flight together share their
// operands' k slabs in L2.
//
// Epilogue: the loads it needs (cos/sin of the tile's tokens, their cache
// rows, the biases) are all issued before the first use -- the cos/sin slice
// straight into the LDS ring, which is free by then -- so a tile's epilogue
// waits for memory once instead of once per token group.
namespace mm {
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLdsMax = 160 * 1024;           // per workgroup on gfx950

// HD, the tile shape (MI token tiles and G pair groups per wave, WN waves
// along the outputs), the k depth BK of a stage (32, 64 or 128) and the
// weight format (W8: one-byte E4M3 weights, so a weight row of a stage is
// half as long as a token row)
template <int HD, int MI, int WN, int BK, int G, bool W8>
struct Shape {
    static constexpr int WM = kWaves / WN;
    static constexpr int BM = WM * MI * 32;
    static constexpr int BN = WN * G * 64;
    static constexpr int kRow = BK * 2;           // bytes per token row and stage
    static constexpr int kCpr = BK / 8;           // 16-byte chunks per token row
    static constexpr int kRpi = 1024 / kRow;      // token rows per load instruction
    static constexpr int kRowB = W8 ? BK : BK * 2;  // the same for the weight rows
    static constexpr int kCprB = kRowB / 16;
    static constexpr int kRpiB = 1024 / kRowB;
    static constexpr int KS = BK / 16;            // k steps of 16 per stage
    static constexpr int kRegionA = BM * kRow;
    static constexpr int kStage = kRegionA + BN * kRowB;
    // ring depth: as many stages as the LDS holds, at most 4
    static constexpr int NSTAGE = kLdsMax / kStage >= 4 ? 4 : kLdsMax / kStage;
    static constexpr int kRing = NSTAGE * kStage;
    // load instructions per stage: an equal share per wave when there are 8
    // or more, else (4 of them) token rows on waves 0-3 and weight rows on
    // waves 4-7
    static constexpr int kInstA = BM / kRpi, kInstB = BN / kRpiB;
    static constexpr int kWaveA = kInstA >= kWaves ? kInstA / kWaves : 1;
    static constexpr int kWaveB = kInstB >= kWaves ? kInstB / kWaves : 1;
    // loads per stage of waves 0-3 and of waves 4-7
    static constexpr int kLoadsLo = kWaveA + (kInstB >= kWaves ? kWaveB : 0);
    static constexpr int kLoadsHi = (kInstA >= kWaves ? kWaveA : 0) + kWaveB;
    // epilogue: every pair index of the head (either pairing reads any of
    // them) as cos then sin per token, in 16-byte chunks
    static constexpr int kPW = HD / 2;
    static constexpr int kChunks = kPW / 2;
    static constexpr int kTab = BM * kChunks * 16;
    // W8: the tile's row scales after the table, [pair group][lo | partner][32]
    static constexpr int kScl = W8 ? BN * 4 : 0;
    static constexpr int kLds = kRing > kTab + kScl ? kRing : kTab + kScl;
    static_assert(BK == 32 || BK == 64 || BK == 128, "stage depth");
    static_assert(!W8 || BK >= 64, "E4M3 weights: stages 64 or 128 deep");
    static_assert(NSTAGE >= 2, "the LDS holds two stages");
    static_assert(kInstA % kWaves == 0 || kInstA == 4, "token-row loads");
    static_assert(kInstB % kWaves == 0 || kInstB == 4, "weight-row loads");
    static_assert(kInstA >= kWaves || kInstB >= kWaves, "load split");
    static_assert(kWaveA <= 8 && kWaveB <= 8, "load slots");
    static_assert((NSTAGE - 1) * (kLoadsLo > kLoadsHi ? kLoadsLo : kLoadsHi) <= 63, "vmcnt range");
    static_assert((BM * kChunks) % 64 == 0, "table staging");
    static_assert(kLds <= kLdsMax, "LDS");
};

// Word 3 of a raw buffer resource (32-bit data format, no swizzle, no
// index stride): untyped loads of the byte range [base, base + num_records).
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediate that waits for vmcnt <= v only
constexpr int vmcnt_wait(int v)
{
    return (v & 15) | ((v >> 4) << 14) | (0xF << 8) | (7 << 4);
}

// Meet the other waves once this wave's LDS reads have returned (the caller
// has waited for its own loads into the stage the waves read next).  The
// empty asm statements keep the compiler from moving memory accesses across
// the barrier; __syncthreads() would also do that, but its fence makes the
// compiler wait for every global->LDS load in flight, the stages still
// being prefetched included.
__device__ __forceinline__ void ring_barrier()
{
    __builtin_amdgcn_s_waitcnt((0xF) | (3 << 14) | (7 << 4));   // lgkmcnt(0) only
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Slot of chunk c of row r: c ^ swz(r).  Chosen per row size with a probe
// that replays the fragment reads under rocprofv3 (16 consecutive rows of a
// quarter wave, one chunk each): 4 LDS cycles per ds_read_b128 and no
// bank-conflict cycles for 64-byte rows with (r >> 2) & 3, 128-byte rows
// with (r >> 1) & 7 and 256-byte rows with r & 15; ((r >> 1) ^ (r >> 3)) & 3,
// conflict-free on paper for 64-byte rows, takes 8 cycles.
template <int CPR>
__device__ __forceinline__ int swz(int r)
{
    constexpr int shift = CPR == 4 ? 2 : (CPR == 8 ? 1 : 0);
    return (r >> shift) & (CPR - 1);
}

// first 32-column MFMA tile of NeoX pair group g (its partner is lo + PT)
template <int PT>
__device__ __forceinline__ int group_lo(int g)
{
    return (g / PT) * (2 * PT) + g % PT;
}
}  // namespace mm

// IL: interleaved pairs (2i, 2i+1), else NeoX (j, j + hd/2); a template
// argument so that the NeoX instance carries no code of the other rotation.
// W8: E4M3 weights.  Their bytes go to LDS as they are (a stage's weight row
// is BK bytes); each k step turns the lane's 8 codes into 8 bf16 (exact:
// every E4M3 value is a bf16 value; one 16-byte LDS read serves two steps),
// so the products and the f32 sums are those of bf16 weights; the epilogue
// multiplies each sum by its row's scale before the bias.
template <bool F16, int HD, int MI, int WN, int BK, int G, bool IL, bool W8>
__global__ __launch_bounds__(mm::kThreads) void proj_mfma_kernel(ProjParams p)
{
    using namespace mm;
    using S = Shape<HD, MI, WN, BK, G, W8>;
    constexpr int BM = S::BM;
    constexpr int NSTAGE = S::NSTAGE, KS = S::KS, kRow = S::kRow, kRowB = S::kRowB;
    constexpr int64_t kWel = W8 ? 1 : 2;          // bytes per weight
    constexpr int HALF = HD / 2;
    constexpr int PT = HALF / 32;                 // tile distance of NeoX partners
    extern __shared__ __align__(16) unsigned char lds[];
    typedef __attribute__((address_space(3))) void lds_t;

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int lrow = lane / S::kCpr, slot = lane % S::kCpr;
    const int lrowb = lane / S::kCprB, slotb = lane % S::kCprB;
    const int lr = lane & 31, hi = lane >> 5;

    constexpr int GT = WN * G;                    // pair groups per tile
    const int ng = p.N / 64;                      // NeoX pair groups (64 columns each)
    const int ntn = (ng + GT - 1) / GT;
    const int ntm = (p.M + BM - 1) / BM;
    const int tiles = ntn * ntm;
    const int tile = (int)blockIdx.x % tiles;
    const int split = (int)blockIdx.x / tiles;
    const int m0 = (tile / ntn) * BM;
    const int tn = tile % ntn;
    const int KTall = p.K / BK;
    const int kbeg = (int)((int64_t)split * KTall / p.ksplit);
    const int len = (int)((int64_t)(split + 1) * KTall / p.ksplit) - kbeg;

    // this wave's load instructions: token rows arow[j] (kRpi rows each,
    // lane / kCpr the row within) and weight rows brow[j] (kRpiB rows, lane /
    // kCprB) of the tile; byte offsets from x and from the weight matrix of
    // the load's section (the rows of a load lie in one 32-column tile, so in
    // one section: its base is wave-uniform), each < 2 GiB; rows past the end
    // repeat the last one.  (fixed-size arrays: with a size that depends on
    // the template arguments, captured by the lambda below, hipcc's host pass
    // silently emitted no launch stub)
    const bool do_a = S::kInstA >= kWaves || wave < S::kInstA;
    const bool do_b = S::kInstB >= kWaves || wave >= kWaves - S::kInstB;
    int arow[8] = {0, 0, 0, 0, 0, 0, 0, 0}, brow[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t aoff[8], boff[8];
    int bsec[8];                                  // section of weight load j (wave-uniform)
#pragma unroll
    for (int j = 0; j < S::kWaveA; ++j) {
        arow[j] = S::kRpi * ((S::kInstA >= kWaves ? wave * S::kWaveA : wave) + j);
        const int r = arow[j] + lrow;
        aoff[j] = (uint32_t)((int64_t)min(m0 + r, p.M - 1) * p.ld_x * 2) + (slot ^ swz<S::kCpr>(r)) * 16;
    }
#pragma unroll
    for (int j = 0; j < S::kWaveB; ++j) {
        brow[j] = S::kRpiB * ((S::kInstB >= kWaves ? wave * S::kWaveB : wave - (kWaves - S::kInstB)) + j);
        const int rb = brow[j] + lrowb;
        const int n = group_lo<PT>(tn * GT + rb / 64) * 32 + ((rb >> 5) & 1) * PT * 32 + (rb & 31);
        const int nu = group_lo<PT>(tn * GT + brow[j] / 64) * 32 + ((brow[j] >> 5) & 1) * PT * 32;
        const int sec = nu < p.nqt ? 0 : (nu < p.nqt + p.nkt ? 1 : 2);
        const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
        bsec[j] = sec;
        boff[j] = (uint32_t)((int64_t)(min(n, p.N - 1) - sbase) * p.K * kWel) + (slotb ^ swz<S::kCprB>(rb)) * 16;
    }
    // buffer resources over x and the three weight matrices: the loads take a
    // 32-bit offset from a scalar base (as fast as 64-bit per-lane addresses
    // or up to 2% faster, 256-4096 tokens), and the hardware clamps them to
    // each buffer's byte range (a load past it would read zeros, never fault)
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(p.x), (short)0,
                                          (int)(((int64_t)(p.M - 1) * p.ld_x + p.K) * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.wsec[0]), (short)0, (int)((int64_t)p.nqt * p.K * kWel), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.wsec[1]), (short)0, (int)((int64_t)p.nkt * p.K * kWel), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw2 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(p.wsec[2]), (short)0, (int)((int64_t)p.nkt * p.K * kWel), kRsrcWord3);
    // local stage st (clamped to the last one: the loop stays uniform)
    auto issue = [&](int st) {
        const int stage = st % NSTAGE;
        const uint32_t kst = (uint32_t)(kbeg + min(st, len - 1));
        const uint32_t kb = kst * kRow, kbb = kst * kRowB;
        unsigned char *sa = lds + stage * S::kStage;
        unsigned char *sb = sa + S::kRegionA;
        if (do_a) {
#pragma unroll
            for (int j = 0; j < S::kWaveA; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_t *)(sa + arow[j] * kRow), 16, aoff[j] + kb, 0,
                                                         0, 0);
        }
        if (do_b) {
#pragma unroll
            for (int j = 0; j < S::kWaveB; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(bsec[j] == 0 ? rw0 : (bsec[j] == 1 ? rw1 : rw2),
                                                         (lds_t *)(sb + brow[j] * kRowB), 16, boff[j] + kbb, 0, 0,
                                                         0);
        }
    };

    // acc[(2g + f) * MI + ti]: output tile f (0: lo, 1: partner) of the
    // wave's pair group g x token tile ti
    f32x16 acc[2 * G * MI];
#pragma unroll
    for (int q = 0; q < 2 * G * MI; ++q)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[q][v] = 0.0f;

    // fragment reads: lane reads row lr of each 32-row tile, chunk 2j + hi
    // for k step j of the stage.  W8: the k values inside a stage are taken
    // in another order (the same for both operands, so only the order of
    // the f32 sums changes): lane (lr, hi) of steps 2p and 2p + 1 takes the
    // 16 codes of weight chunk 2p + hi, one 16-byte read for the step pair
    // (8-byte reads of the 64-byte E4M3 rows reach only half the banks per
    // half-wave), and its token chunks 4p + 2hi and 4p + 2hi + 1.
    const int g = swz<S::kCpr>(lr);               // tiles start at multiples of 32
    const int gb = swz<S::kCprB>(lr);
    const int abase = (wm * MI * 32 + lr) * kRow;
    const int bbase = S::kRegionA + (wn * G * 64 + lr) * kRowB;
    int koff[8], koffb[4];
#pragma unroll
    for (int j = 0; j < KS; ++j)
        koff[j] = ((W8 ? 4 * (j >> 1) + 2 * hi + (j & 1) : 2 * j + hi) ^ g) * 16;
#pragma unroll
    for (int q = 0; q < KS / 2; ++q)
        koffb[q] = ((2 * q + hi) ^ gb) * 16;
    u32x4 braw[6];                                // W8: a step pair's codes, per weight tile
    // two fragment buffers: step j uses buffer j % 2
    static_assert(KS % 2 == 0, "steps per stage");
    bf16x8 a0[MI], b0[2 * G], a1[MI], b1[2 * G];
    // bf16: the reads go out in the order the products first use them (the
    // first weight fragment, the token fragments, the other weight fragments)
    auto read_frags = [&](const unsigned char *s, int j, bf16x8 (&fa)[MI], bf16x8 (&fb)[2 * G]) {
        if constexpr (!W8)
            fb[0] = *reinterpret_cast<const bf16x8 *>(s + bbase + koff[j]);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            fa[mi] = *reinterpret_cast<const bf16x8 *>(s + abase + mi * 32 * kRow + koff[j]);
#pragma unroll
        for (int t = W8 ? 0 : 1; t < 2 * G; ++t) {
            if constexpr (W8) {
                // even step: read the pair's 16 codes, convert the first 8;
                // odd step: convert the other 8 (no LDS read)
                if ((j & 1) == 0)
                    braw[t] = *reinterpret_cast<const u32x4 *>(s + bbase + t * 32 * kRowB + koffb[j >> 1]);
                const unsigned int c0 = (j & 1) ? braw[t].z : braw[t].x;
                const unsigned int c1 = (j & 1) ? braw[t].w : braw[t].y;
                const bf16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, 1.0f, false);
                const bf16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c0, 1.0f, true);
                const bf16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, 1.0f, false);
                const bf16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c1, 1.0f, true);
                fb[t] = __builtin_shufflevector(__builtin_shufflevector(w0, w1, 0, 1, 2, 3),
                                                __builtin_shufflevector(w2, w3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                fb[t] = *reinterpret_cast<const bf16x8 *>(s + bbase + t * 32 * kRowB + koff[j]);
            }
        }
    };
    // half h takes products q = (2g + f)*MI + ti in [h*G*MI, (h+1)*G*MI)
    auto mfma_half = [&](int h, const bf16x8 (&fa)[MI], const bf16x8 (&fb)[2 * G]) {
#pragma unroll
        for (int q = h * G * MI; q < (h + 1) * G * MI; ++q)
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[q / MI], fa[q % MI], acc[q], 0, 0, 0);
    };

    // The next step's fragment reads, spread over this step's products: one
    // LDS read after each MFMA while both last (sched_group_barrier masks:
    // 0x008 MFMA, 0x100 LDS read).  Every read then has about seven MFMAs in
    // front of its first use, and the eight waves' reads reach the LDS spread
    // over the step instead of in one burst after its first half.
    auto spread_reads = [&]() {
        constexpr int kM = 2 * G * MI, kR = W8 ? MI : MI + 2 * G;
#pragma unroll
        for (int i = 0; i < (kR < kM ? kR : kM); ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (kM > kR)
            __builtin_amdgcn_sched_group_barrier(0x008, kM - kR, 0);
    };

    // prologue: stages 0..NSTAGE-1 in flight, stage 0 landed everywhere
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st)
        issue(st);
    if (S::kLoadsLo == S::kLoadsHi || wave < 4)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait((NSTAGE - 1) * S::kLoadsLo));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait((NSTAGE - 1) * S::kLoadsHi));
    ring_barrier();
    read_frags(lds, 0, a0, b0);

    // Per pair of k steps: step j's products with the fragment reads of step
    // j + 1 spread among them; then step j + 1's products with those of step
    // j + 2 -- or, after the stage's last step: its first half, then wait
    // for this wave's loads of the next stage, meet the other waves (after
    // which this stage is free and the next visible), refill this stage
    // NSTAGE ahead, read the next stage's first fragments, and the second
    // half.  The refill goes out right after the barrier: with two stages
    // (256 x 256) it has one stage's time to land, and issuing it later,
    // even spread between the products, measured slower.
    for (int kt = 0; kt < len; ++kt) {
        const unsigned char *s = lds + (kt % NSTAGE) * S::kStage;
        // steps in pairs (KS is even): step jj on buffer 0, jj + 1 on buffer 1
#pragma unroll
        for (int jj = 0; jj < KS; jj += 2) {
            __builtin_amdgcn_sched_barrier(0);
            mfma_half(0, a0, b0);
            read_frags(s, jj + 1, a1, b1);
            mfma_half(1, a0, b0);
            spread_reads();
            __builtin_amdgcn_sched_barrier(0);
            if (jj + 2 < KS) {
                mfma_half(0, a1, b1);
                read_frags(s, jj + 2, a0, b0);
                mfma_half(1, a1, b1);
                spread_reads();
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfma_half(0, a1, b1);
                __builtin_amdgcn_sched_barrier(0);
                if (S::kLoadsLo == S::kLoadsHi || wave < 4)
                    __builtin_amdgcn_s_waitcnt(vmcnt_wait((NSTAGE - 2) * S::kLoadsLo));
                else
                    __builtin_amdgcn_s_waitcnt(vmcnt_wait((NSTAGE - 2) * S::kLoadsHi));
                ring_barrier();
                issue(kt + NSTAGE);
                read_frags(lds + ((kt + 1) % NSTAGE) * S::kStage, 0, a0, b0);
                __builtin_amdgcn_sched_barrier(0);
                mfma_half(1, a1, b1);
            }
        }
    }
    // the clamped reloads of the last iterations land before the ring is
    // reused or the workgroup leaves
    __builtin_amdgcn_s_waitcnt(0);

    // Lane (lr, hi) holds, for token ti*32 + lr of the wave's tokens and its
    // pair group g, the outputs col0[g] + f*HALF + 8gg + 4hi + e (e < 4) in
    // acc[(2g + f)*MI + ti][4gg + e]: four consecutive columns; f = 1 is the
    // NeoX partner of f = 0.
    int col0[G];
    bool live[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int gi = tn * GT + wn * G + g;
        live[g] = gi < ng;
        col0[g] = group_lo<PT>(gi) * 32;
    }
    const int tok0 = m0 + wm * MI * 32 + lr;     // token of ti = 0
    if (p.ksplit > 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!live[g])
                continue;
            float *const out = p.part + (int64_t)split * p.M * p.N + col0[g] + 4 * hi;
#pragma unroll
            for (int ti = 0; ti < MI; ++ti) {
                const int tok = tok0 + ti * 32;
                if (tok >= p.M)
                    continue;
                float *const orow = out + (int64_t)tok * p.N;
#pragma unroll
                for (int f = 0; f < 2; ++f)     // half by half: whole 128-byte lines
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg) {
                        const f32x16 &av = acc[(2 * g + f) * MI + ti];
                        const FVec<4> y = {{av[4 * gg], av[4 * gg + 1], av[4 * gg + 2], av[4 * gg + 3]}};
                        st_data<4, false>(orow + f * HALF + 8 * gg, y);
                    }
            }
        }
        return;
    }

    // ---- epilogue ---------------------------------------------------------
    // Stage the cos/sin table rows of the tile's BM tokens into the LDS ring:
    // chunk c of token r in slot c ^ (r % kChunks), which keeps the reads
    // below (32 tokens, one chunk) conflict-free.
    __syncthreads();                              // every wave is done with the ring
    {
        constexpr int kInst = BM * S::kChunks / 64;
        for (int u = wave; u < kInst; u += kWaves) {
            const int ca = u * 64 + lane;
            const int r = ca / S::kChunks, sl = ca % S::kChunks;
            const int c = sl ^ (r % S::kChunks);
            const int tokc = min(m0 + r, p.M - 1);
            const int col = 4 * c;                    // cos chunks, then sin
            __builtin_amdgcn_global_load_lds(p.rtab + (int64_t)tokc * HD + col, (lds_t *)(lds + u * 1024), 16, 0,
                                             0);
        }
        if constexpr (W8) {
            // thread u < GT*16 copies 16 bytes: pair group q = u / 16, its lo
            // (f = 0) or partner (f = 1) columns, four of them; a group past
            // the last output is not read below
            const int u = tid;
            const int q = u >> 4, f = (u >> 3) & 1, c4 = (u & 7) * 4;
            if (u < GT * 16 && tn * GT + q < ng) {
                const float *const src = p.wscale + group_lo<PT>(tn * GT + q) * 32 + f * HALF + c4;
                float *const dst = reinterpret_cast<float *>(lds + S::kTab) + q * 64 + f * 32 + c4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[e] = src[e];
            }
        }
    }
    // per pair group: its section, the lane's 32 bias values; the tokens'
    // cache rows when any group is in k or v
    int sec[G], cs[G];
    FVec<4> bias0[G][4], bias1[G][4];
    bool any_kv = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        sec[g] = col0[g] < p.nqt ? 0 : (col0[g] < p.nqt + p.nkt ? 1 : 2);
        const int sbase = sec[g] == 0 ? 0 : (sec[g] == 1 ? p.nqt : p.nqt + p.nkt);
        cs[g] = col0[g] - sbase + 4 * hi;         // section column of (f = 0, gg = 0)
        any_kv = any_kv || (live[g] && sec[g] > 0);
        const float *const bias = live[g] ? p.b[sec[g]] : nullptr;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            if (bias && p.vec) {
                bias0[g][gg] = ld_vec<4>(bias + cs[g] + 8 * gg);
                bias1[g][gg] = ld_vec<4>(bias + cs[g] + 8 * gg + HALF);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bias0[g][gg].e[e] = bias ? bias[cs[g] + 8 * gg + e] : 0.0f;
                    bias1[g][gg].e[e] = bias ? bias[cs[g] + 8 * gg + e + HALF] : 0.0f;
                }
            }
        }
    }
    int64_t crow[MI];
#pragma unroll
    for (int ti = 0; ti < MI; ++ti)
        crow[ti] = any_kv ? p.rows[min(tok0 + ti * 32, p.M - 1)] : -1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (!live[g])
            continue;
        float *const out = p.out[sec[g]];
        const int64_t ldo = p.ld[sec[g]];
        void *const cache = sec[g] == 1 ? p.cache[0] : p.cache[1];
        const int cpair = (col0[g] % HD) / 4 + hi;   // cos chunk of (gg = 0)
#pragma unroll
        for (int ti = 0; ti < MI; ++ti) {
            const int tok = tok0 + ti * 32;
            if (tok >= p.M)
                continue;
            const int r = tok - m0;
            const int64_t row = sec[g] > 0 ? crow[ti] : -1;
            float *const orow = out + (int64_t)tok * ldo;
            const unsigned char *trow = lds + r * S::kChunks * 16;
            // the lane's 16 outputs of each half, rotated, then stored half by
            // half: four consecutive stores complete the wave's 128-byte lines
            // of a row, so the L2 merges each line from back-to-back writes
            // (0-2% faster at 2048-4096 tokens than interleaving the halves)
            FVec<4> Y0[4], Y1[4];
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int c0 = cs[g] + 8 * gg, c1 = c0 + HALF;
                FVec<4> &y0 = Y0[gg], &y1 = Y1[gg];
                if constexpr (W8) {
                    // each sum times its row's scale, rounded, then the bias
                    // (two roundings, as the weight-streaming kernel: no FMA)
#pragma clang fp contract(off)
                    const float *const sl = reinterpret_cast<const float *>(lds + S::kTab) +
                                            (wn * G + g) * 64 + 8 * gg + 4 * hi;
                    const FVec<4> sc0 = *reinterpret_cast<const FVec<4> *>(sl);
                    const FVec<4> sc1 = *reinterpret_cast<const FVec<4> *>(sl + 32);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float m0 = acc[2 * g * MI + ti][4 * gg + e] * sc0.e[e];
                        const float m1 = acc[(2 * g + 1) * MI + ti][4 * gg + e] * sc1.e[e];
                        y0.e[e] = m0 + bias0[g][gg].e[e];
                        y1.e[e] = m1 + bias1[g][gg].e[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        y0.e[e] = acc[2 * g * MI + ti][4 * gg + e] + bias0[g][gg].e[e];
                        y1.e[e] = acc[(2 * g + 1) * MI + ti][4 * gg + e] + bias1[g][gg].e[e];
                    }
                }
                if (sec[g] < 2 && !IL) {
                    const int cc = cpair + 2 * gg;
                    const FVec<4> cv = *reinterpret_cast<const FVec<4> *>(trow + ((cc ^ (r % S::kChunks)) * 16));
                    const FVec<4> sv = *reinterpret_cast<const FVec<4> *>(
                        trow + (((cc + S::kChunks / 2) ^ (r % S::kChunks)) * 16));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        rot(y0.e[e], y1.e[e], cv.e[e], sv.e[e]);
                } else if (sec[g] < 2) {
                    // interleaved pairs (2i, 2i+1) sit in the lane's own four
                    // columns: pair indices pi, pi + 1 with pi = 2hi (mod 4),
                    // so elements 2hi, 2hi + 1 of one 16-byte chunk (chosen
                    // by select: an indexed register read would go to scratch)
#pragma unroll
                    for (int f = 0; f < 2; ++f) {
                        FVec<4> &y = f ? y1 : y0;
                        const int pi = ((col0[g] + f * HALF + 8 * gg + 4 * hi) % HD) / 2;
                        const int cc = pi / 4;
                        const FVec<4> cv = *reinterpret_cast<const FVec<4> *>(trow + ((cc ^ (r % S::kChunks)) * 16));
                        const FVec<4> sv = *reinterpret_cast<const FVec<4> *>(
                            trow + (((cc + S::kChunks / 2) ^ (r % S::kChunks)) * 16));
                        rot(y.e[0], y.e[1], hi ? cv.e[2] : cv.e[0], hi ? sv.e[2] : sv.e[0]);
                        rot(y.e[2], y.e[3], hi ? cv.e[3] : cv.e[1], hi ? sv.e[3] : sv.e[1]);
                    }
                }
                if (!p.vec) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        orow[c0 + e] = y0.e[e];
                        orow[c1 + e] = y1.e[e];
                        if (row >= 0) {
                            put_cache<F16>(cache, row * p.nkt + c0 + e, y0.e[e]);
                            put_cache<F16>(cache, row * p.nkt + c1 + e, y1.e[e]);
                        }
                    }
                }
            }
            if (p.vec) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int gg = 0; gg < 4; ++gg)
                        st_data<4, false>(orow + cs[g] + 8 * gg + f * HALF, f ? Y1[gg] : Y0[gg]);
                if (row >= 0) {
#pragma unroll
                    for (int f = 0; f < 2; ++f)
#pragma unroll
                        for (int gg = 0; gg < 4; ++gg)
                            st_cache<4, F16, false>(cache, row * p.nkt + cs[g] + 8 * gg + f * HALF,
                                                    f ? Y1[gg] : Y0[gg]);
                }
            }
            if (sec[g] > 0 && row < 0 && hi == 0)
                atomicOr(p.err, 1u);
        }
    }
}

// ---------------------------------------------------------------------------
// split path, second step: y = sum of the k-split partials (in split order,
// so the result does not depend on timing), then the epilogue.  A thread
// takes pair index i of token t in hpt consecutive heads (the v section
// pairs its columns the same way, without the rotation): it computes the
// pair's cos/sin (f32 angle, double sincos rounded to f32, as the table of
// the fused path) and the token's cache row once for all of them; hpt grows
// with the batch only as far as keeps ~256K threads in flight (fewer, longer
// threads measured slower: 54 against 50 us at 256 tokens with 115K).  A wave covers
// consecutive i of one (token, head group), so the partials are read in
// 256-byte runs.
// ---------------------------------------------------------------------------
int split_heads_per_thread(int M, int N, int hd)
{
    const int64_t pairs = (int64_t)M * (N / 2);
    int hpt = 1;
    while (hpt < 8 && pairs / (hpt * 2) >= 262144)
        hpt *= 2;
    return hpt;
}

template <bool F16, int HD>
__global__ __launch_bounds__(256) void proj_split_epilogue_kernel(ProjParams p, InvTableSmall inv, int hpt)
{
    constexpr int HALF = HD / 2;
    const int heads = p.N / HD;
    const int groups = (heads + hpt - 1) / hpt;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * groups * HALF)
        return;
    const int i = (int)(idx % HALF);
    const int64_t rest = idx / HALF;
    const int hg = (int)(rest % groups);
    const int t = (int)(rest / groups);
    const int h0 = hg * hpt;
    const int h1 = min(h0 + hpt, heads);
    const int qheads = p.nqt / HD, kheads = p.nkt / HD;
    float cv = 1.0f, sv = 0.0f;
    if (h0 < qheads + kheads) {
        const float ang = (float)p.pos[t] * inv.v[i];
        double sd, cd;
        sincos((double)ang, &sd, &cd);
        cv = (float)cd;
        sv = (float)sd;
    }
    const int64_t row = h1 > qheads ? cache_row(p, t) : -1;
    const int64_t plane = (int64_t)p.M * p.N;
    const float *const srow = p.part + (int64_t)t * p.N;
    const bool il = p.style == QKV_ROPE_INTERLEAVED;
    for (int h = h0; h < h1; ++h) {
        // pair i: columns (i, i + hd/2) of the head, interleaved (2i, 2i + 1)
        const int c0 = h * HD + (il ? 2 * i : i), c1 = c0 + (il ? 1 : HALF);
        const float *src = srow;
        float y0 = src[c0], y1 = src[c1];
#pragma unroll 4
        for (int sp = 1; sp < p.ksplit; ++sp) {
            src += plane;
            y0 = y0 + src[c0];
            y1 = y1 + src[c1];
        }
        if (p.w8) {
            y0 = y0 * p.wscale[c0];
            y1 = y1 * p.wscale[c1];
        }
        const int sec = h < qheads ? 0 : (h < qheads + kheads ? 1 : 2);
        const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
        const int s0 = c0 - sbase, s1 = c1 - sbase;
        const float *bias = p.b[sec];
        if (bias) {
            y0 = y0 + bias[s0];
            y1 = y1 + bias[s1];
        }
        if (sec < 2)
            rot(y0, y1, cv, sv);
        float *out = p.out[sec] + (int64_t)t * p.ld[sec];
        out[s0] = y0;
        out[s1] = y1;
        if (sec > 0) {
            void *cache = sec == 1 ? p.cache[0] : p.cache[1];
            if (row >= 0) {
                put_cache<F16>(cache, row * p.nkt + s0, y0);
                put_cache<F16>(cache, row * p.nkt + s1, y1);
            } else if (i == 0) {          // one lane per head reports the token
                atomicOr(p.err, 1u);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// decode (1-4 tokens): weight-streaming GEMV + epilogue
// ---------------------------------------------------------------------------
// kGemvSplit waves per NeoX pair of weight rows (j and j + hd/2 of a head; in
// the v section the same pairing just groups rows), each over its share of
// k, four waves per block.  Lane l takes the 16-byte chunks l, l+64, ... of
// the wave's share of both rows, U chunks in flight per row, and keeps NT
// running sums per row (v_dot2_f32_bf16: two bf16 products into the f32 sum
// per instruction); a butterfly over the wave completes its part of the dot
// products, the pair's first wave adds the others' through LDS in k order,
// and its lane t < nt finishes token t: bias, the rotation of the pair,
// write-back and the cache store.  Two waves per pair (twice the waves in
// flight, one step each at 14B) measured 13.9 -> 13.1 us per 14B layer.
// up to 4 tokens; from 5 the k-split MFMA path is faster (5-8 tokens: 21.7-
// 21.9 us at 14B against 24.6-24.9 for a GEMV with four pairs per wave)
constexpr int kGemvTok = 4;
constexpr int kGemvWaves = 4;     // waves per block
constexpr int kGemvSplit = 2;     // waves per NeoX pair, each summing 1/kGemvSplit of k

// U: 16-byte chunks of each row in flight per lane and step; the launcher
// picks U dividing the chunks per lane (hidden/512) when it can, since a
// partial last step costs as much as a full one.  P: pairs per wave (1,
// except 2 for 4 tokens of E4M3 weights at hidden >= 4096; more pairs let
// one x chunk serve more weight rows; P divides the pair count N/2, a
// multiple of 64).
// SEP: q, k, v weights in three matrices (the concat layout keeps its own
// instance: the per-section select cost ~1% at 14B).  W8: E4M3 weights, a
// 16-byte chunk holding 16 of them (two chunks of x); each output is its f32
// sum times the row's scale.
template <bool F16, int HD, int NT, int U, int P, bool SEP, bool W8>
__global__ __launch_bounds__(64 * kGemvWaves) void proj_gemv_kernel(ProjParams p, InvTableSmall inv)
{
    constexpr int HALF = HD / 2;
    constexpr int kWpc = W8 ? 16 : 8;        // weights per 16-byte chunk
    constexpr int XV = kWpc / 8;             // 16-byte chunks of x per weight chunk
    constexpr int R = 2 * P;                 // weight rows per wave
    const int lane = (int)threadIdx.x & 63;
    const int wvi = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int kq = wvi % kGemvSplit;         // this wave's share of k
    const int pair0 = ((int)blockIdx.x * (kGemvWaves / kGemvSplit) + wvi / kGemvSplit) * P;
    const bool valid = pair0 < p.N / 2;      // (every wave reaches the barrier below)
    const int nchunk = p.K / kWpc;           // hidden % 64 == 0: kGemvSplit divides it
    const int c_beg = kq * (nchunk / kGemvSplit);
    const int c_end = valid ? c_beg + nchunk / kGemvSplit : c_beg;
    // rows 2q and 2q+1 are the two columns of pair pair0 + q: c0 and c0 +
    // hd/2 (NeoX) or c0 + 1 (interleaved)
    const bool il = p.style == QKV_ROPE_INTERLEAVED;
    const unsigned char *wr[R];
#pragma unroll
    for (int q = 0; q < P; ++q) {
        const int pr = valid ? pair0 + q : 0;
        const int c0 = (pr / HALF) * HD + (il ? 2 * (pr % HALF) : pr % HALF);
        wr[2 * q] = weight_row<SEP, W8>(p, c0);
        wr[2 * q + 1] = weight_row<SEP, W8>(p, c0 + (il ? 1 : HALF));
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
    for (int cb = c_beg + lane; cb < c_end; cb += 64 * U) {
        u32x4 wv[U][R], xv[U][NT][XV];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = cb + 64 * u;
            ok[u] = c < c_end;
            const int cc = ok[u] ? c : 0;    // past the row end: reload chunk 0, weight 0
            // the weights are read once per call: nontemporal
#pragma unroll
            for (int r = 0; r < R; ++r)
                wv[u][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wr[r] + cc * 16));
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < XV; ++j)
                    xv[u][t][j] = *reinterpret_cast<const u32x4 *>(xr[t] + cc * kWpc + 8 * j);
        }
        // every load of the step goes out before the first product (left to
        // itself the scheduler interleaved them, waiting on each in turn):
        // 14.3 -> 13.9 us per 14B layer, 10.7 -> 10.4 at hidden 3584
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // each dword holds two consecutive bf16 of a row (x and W alike):
            // one dot2 adds both exact products to the f32 sum.  The pairs are
            // taken from the whole 16-byte vector by shuffles: bit-casting
            // single dwords of it compiled to one-dword loads reused for all
            // four pairs (checked in the ISA).
            bf16x8 xx8[NT][XV];
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < XV; ++j)
                    xx8[t][j] = __builtin_bit_cast(bf16x8, xv[u][t][j]);
#define QKV_PAIR(v8, e) __builtin_shufflevector(v8, v8, 2 * (e), 2 * (e) + 1)
            if constexpr (W8) {
                // dword i of the chunk holds weights 4i..4i+3; each half
                // converts to two bf16 (exact: every E4M3 value is one) and
                // meets x elements 4i.. of the chunk's two x chunks
#define QKV_W8_DWORD(i, j, e)                                                                          \
    {                                                                                                  \
        const bf16x2 wlo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[i], 1.0f, false);              \
        const bf16x2 whi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[i], 1.0f, true);               \
        for (int t = 0; t < NT; ++t) {                                                                 \
            d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][j], e), wlo, d[r][t], false);     \
            d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][j], e + 1), whi, d[r][t], false); \
        }                                                                                              \
    }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u32x4 wq = ok[u] ? wv[u][r] : u32x4{0u, 0u, 0u, 0u};
                    QKV_W8_DWORD(0, 0, 0)
                    QKV_W8_DWORD(1, 0, 2)
                    QKV_W8_DWORD(2, XV - 1, 0)
                    QKV_W8_DWORD(3, XV - 1, 2)
                }
#undef QKV_W8_DWORD
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const bf16x8 w8 = __builtin_bit_cast(bf16x8, ok[u] ? wv[u][r] : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][0], 0), QKV_PAIR(w8, 0), d[r][t], false);
                        d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][0], 1), QKV_PAIR(w8, 1), d[r][t], false);
                        d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][0], 2), QKV_PAIR(w8, 2), d[r][t], false);
                        d[r][t] = __builtin_amdgcn_fdot2_f32_bf16(QKV_PAIR(xx8[t][0], 3), QKV_PAIR(w8, 3), d[r][t], false);
                    }
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
    // the pair's first wave adds the other waves' sums in k order
    __shared__ float part[kGemvWaves][R][NT];
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                part[wvi][r][t] = d[r][t];
    }
    __syncthreads();
    if (kq != 0 || !valid)
        return;
#pragma unroll
    for (int s = 1; s < kGemvSplit; ++s)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                d[r][t] += part[wvi + s][r][t];

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
        const int c0 = (pr / HALF) * HD + (il ? 2 * i : i);   // global output column of the pair's first row
        const int sec = c0 < p.nqt ? 0 : (c0 < p.nqt + p.nkt ? 1 : 2);
        const int sbase = sec == 0 ? 0 : (sec == 1 ? p.nqt : p.nqt + p.nkt);
        const int s0 = c0 - sbase, s1 = s0 + (il ? 1 : HALF);   // columns inside the section
        if (W8) {
            y0 = y0 * p.wscale[c0];
            y1 = y1 * p.wscale[c0 + (s1 - s0)];
        }
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

// Launch choice.  Decode (1-4 tokens): the GEMV.  5+ tokens: the per-launch
// tables, then the MFMA kernel on the tile shape and k split chosen below,
// and the summing epilogue when k is split.
struct MmPlan {
    int mi, wn, g;           // token tiles and pair groups per wave, waves along the outputs
    int ksplit;
};

int mm_bm(int mi, int wn)
{
    return mm::kWaves / wn * mi * 32;
}

// Tile shape and k split: the plan the cost model below rates fastest.  Per
// stage of k (64) a workgroup of each shape takes, measured on MI355X with
// every CU busy (14B q|k|v, hidden 5120; epilogue included): 256 x 256 1.9
// us, 256 x 192 1.58, 256 x 128 1.13, 128 x 128 0.72, 64 x 256 0.9.  A launch
// runs ceil(tiles * S / CUs) rounds of K/64/S stages; it cannot beat
// streaming the weights once from HBM (~5.5 TB/s with every CU pulling its
// share, less with fewer workgroups than CUs); a k split adds the round trip
// of its S*M*N f32 partials (~5 TB/s) and a summing kernel (~3 us), no split
// the cos/sin table kernel (~4 us).  Against sweeps of every shape and split
// at 16-4096 tokens it picks the fastest measured plan or one within 3%.
MmPlan mm_plan(int M, int N, int K, int cus, bool w8)
{
    struct Cand {
        int mi, wn, g;
        double us;                                  // per stage of 64
    };
    static const Cand cands[5] = {
        {4, 4, 1, 1.90}, {2, 2, 1, 1.13}, {1, 2, 1, 0.72}, {1, 4, 1, 0.90}, {1, 1, 3, 1.58}};
    const int KT = K / 64;
    const int NG = N / 64;
    const double w_us = (double)N * K * (w8 ? 1 : 2) / 5.5e6;
    MmPlan best = {4, 4, 1, 1};
    double best_t = 1e300;
    for (const Cand &c : cands) {
        if (w8 && c.g == 3)
            continue;   // 12 weight-row loads per E4M3 stage do not share out over 8 waves
        const int64_t bm = mm_bm(c.mi, c.wn), gt = c.wn * c.g;
        const int64_t tiles = ((M + bm - 1) / bm) * ((NG + gt - 1) / gt);
        const int smax = KT / 4 < 1 ? 1 : (KT / 4 > 64 ? 64 : KT / 4);   // >= 4 stages per split
        for (int ks = 1; ks <= smax; ++ks) {
            if (ks > 1 && tiles * (ks - 1) >= cus)  // a split beyond filling the chip
                break;
            const double rounds = (double)((tiles * ks + cus - 1) / cus);
            const double busy = (double)std::min<int64_t>(tiles * ks, cus) / cus;
            double t = std::max(rounds * ((double)KT / ks) * c.us, w_us / busy);
            t += ks > 1 ? 2.0 * ks * (double)M * N * 4 / 5.0e6 + 3.0 : 4.0;
            if (t < best_t) {
                best_t = t;
                best = {c.mi, c.wn, c.g, ks};
            }
        }
    }
    return best;
}

// Raise the kernel's dynamic-LDS limit to what it uses, once per kernel and
// device (the caller has made the handle's device current).
template <bool F16, int HD, int MI, int WN, int BK, int G, bool IL, bool W8>
hipError_t set_mm_lds(int device)
{
    static std::atomic<unsigned long long> done{0};
    const unsigned long long bit = 1ull << (device & 63);
    if (done.load(std::memory_order_acquire) & bit)
        return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&proj_mfma_kernel<F16, HD, MI, WN, BK, G, IL, W8>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       mm::Shape<HD, MI, WN, BK, G, W8>::kLds);
    if (e == hipSuccess && device < 64)
        done.fetch_or(bit, std::memory_order_release);
    return e;
}

// chunks per row and step of the GEMV: the largest of 8..4 dividing a
// wave's chunks per lane, else the one wasting the fewest slots
int gemv_step(int K)
{
    const int c = (K / 8 / kGemvSplit + 63) / 64;   // 16-byte chunks per lane and row
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

// the same for E4M3 weights (16 per chunk): the largest of 4..2 dividing the
// chunks per lane, else the one wasting the fewest slots (3 at hidden 5120:
// 160 chunks per wave in one step of 192 slots)
int gemv_step8(int K)
{
    const int c = (K / 16 / kGemvSplit + 63) / 64;
    int best = 2, waste = 1 << 30;
    for (int u = 4; u >= 2; --u) {
        const int w = (c + u - 1) / u * u - c;
        if (w < waste) {
            best = u;
            waste = w;
        }
    }
    return best;
}

template <bool F16, int HD, int NT, bool SEP>
hipError_t launch_gemv(const ProjParams &pp, const InvTableSmall &inv, hipStream_t st, int u)
{
    constexpr int pairs = kGemvWaves / kGemvSplit;   // per block
    const int blocks = (pp.N / 2 + pairs - 1) / pairs;
    const dim3 grid(blocks), block(64 * kGemvWaves);
    if (pp.w8) {
        if constexpr (NT == 4) {
            // 4 tokens at hidden >= 4096: two pairs per wave, so each x chunk
            // serves four weight rows (14B: 15.2 against 15.9 us; at hidden
            // 3584 it measured slower, 9.9 against 9.2)
            if (pp.K >= 4096) {
                const dim3 grid2((blocks + 1) / 2);
                switch (u) {
                case 4: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 4, 2, SEP, true>), grid2, block, 0, st, pp, inv); break;
                case 3: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 3, 2, SEP, true>), grid2, block, 0, st, pp, inv); break;
                default: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 2, 2, SEP, true>), grid2, block, 0, st, pp, inv); break;
                }
                return hipGetLastError();
            }
        }
        switch (u) {
        case 4: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 4, 1, SEP, true>), grid, block, 0, st, pp, inv); break;
        case 3: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 3, 1, SEP, true>), grid, block, 0, st, pp, inv); break;
        default: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 2, 1, SEP, true>), grid, block, 0, st, pp, inv); break;
        }
        return hipGetLastError();
    }
    switch (u) {
    case 8: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 8, 1, SEP, false>), grid, block, 0, st, pp, inv); break;
    case 7: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 7, 1, SEP, false>), grid, block, 0, st, pp, inv); break;
    case 6: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 6, 1, SEP, false>), grid, block, 0, st, pp, inv); break;
    case 5: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 5, 1, SEP, false>), grid, block, 0, st, pp, inv); break;
    default: hipLaunchKernelGGL((proj_gemv_kernel<F16, HD, NT, 4, 1, SEP, false>), grid, block, 0, st, pp, inv); break;
    }
    return hipGetLastError();
}

template <bool F16, int HD, int MI, int WN, int BK, int G, bool IL, bool W8>
hipError_t launch_mm(const ProjParams &pp, hipStream_t st)
{
    using S = mm::Shape<HD, MI, WN, BK, G, W8>;
    hipError_t e = set_mm_lds<F16, HD, MI, WN, BK, G, IL, W8>(pp.device);
    if (e != hipSuccess)
        return e;
    const int gt = WN * G;
    const int tiles = ((pp.M + S::BM - 1) / S::BM) * ((pp.N / 64 + gt - 1) / gt);
    constexpr unsigned lds = S::kLds;
    hipLaunchKernelGGL((proj_mfma_kernel<F16, HD, MI, WN, BK, G, IL, W8>), dim3(tiles * pp.ksplit),
                       dim3(mm::kThreads), lds, st, pp);
    return hipGetLastError();
}

template <bool F16, int HD, bool IL, bool W8>
hipError_t launch_mm_shape(const ProjParams &pp, hipStream_t st, const MmPlan &pl)
{
    switch (pl.mi * 100 + pl.wn * 10 + pl.g) {
    case 141: return launch_mm<F16, HD, 1, 4, 64, 1, IL, W8>(pp, st);
    case 121: return launch_mm<F16, HD, 1, 2, 64, 1, IL, W8>(pp, st);
    case 221: return launch_mm<F16, HD, 2, 2, 64, 1, IL, W8>(pp, st);
    case 441: return launch_mm<F16, HD, 4, 4, 64, 1, IL, W8>(pp, st);
    case 113:
        if constexpr (W8)
            return hipErrorInvalidValue;    // the planner never picks it for E4M3 weights
        else
            return launch_mm<F16, HD, 1, 1, 64, 3, IL, W8>(pp, st);
    default: return hipErrorInvalidValue;
    }
}

template <bool F16, int HD>
hipError_t launch_mm_plan(const ProjParams &pp, hipStream_t st, const MmPlan &pl)
{
    const bool il = pp.style == QKV_ROPE_INTERLEAVED;
    if (pp.w8)
        return il ? launch_mm_shape<F16, HD, true, true>(pp, st, pl)
                  : launch_mm_shape<F16, HD, false, true>(pp, st, pl);
    return il ? launch_mm_shape<F16, HD, true, false>(pp, st, pl)
              : launch_mm_shape<F16, HD, false, false>(pp, st, pl);
}

template <bool F16, int HD>
hipError_t launch_proj(const ProjParams &pp, const InvTableSmall &inv, hipStream_t st, MmPlan pl)
{
    if (pp.M <= kGemvTok) {
        const int u = pp.w8 ? gemv_step8(pp.K) : gemv_step(pp.K);
        if (pp.M == 1)
            return pp.sep ? launch_gemv<F16, HD, 1, true>(pp, inv, st, u)
                          : launch_gemv<F16, HD, 1, false>(pp, inv, st, u);
        if (pp.M == 2)
            return pp.sep ? launch_gemv<F16, HD, 2, true>(pp, inv, st, u)
                          : launch_gemv<F16, HD, 2, false>(pp, inv, st, u);
        return pp.sep ? launch_gemv<F16, HD, 4, true>(pp, inv, st, u)
                      : launch_gemv<F16, HD, 4, false>(pp, inv, st, u);
    }
    // the fused epilogue reads the launch's cos/sin and cache-row tables; the
    // split path's summing kernel computes its own
    if (pp.ksplit == 1) {
        const int64_t n_tab = (int64_t)pp.M * (HD / 2);
        hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n_tab + 255) / 256)), dim3(256), 0, st, pp, inv,
                           const_cast<float *>(pp.rtab), const_cast<int64_t *>(pp.rows));
    }
    hipError_t e = launch_mm_plan<F16, HD>(pp, st, pl);
    if (e != hipSuccess || pp.ksplit == 1)
        return e;
    const int hpt = split_heads_per_thread(pp.M, pp.N, HD);
    const int64_t groups = (pp.N / HD + hpt - 1) / hpt;
    const int64_t n_thr = (int64_t)pp.M * groups * (HD / 2);
    hipLaunchKernelGGL((proj_split_epilogue_kernel<F16, HD>), dim3((unsigned)((n_thr + 255) / 256)),
                       dim3(256), 0, st, pp, inv, hpt);
    return hipGetLastError();
}

}  // namespace

// ---- the workspace of the allocation-free entry point -----------------------
// A file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  Its device address is taken once per device at handle
// creation (proj_scratch_setup) with that device current; host code uses only
// that address, never the array's name (which names a host-side stand-in).
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
void *g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

namespace qkv_detail {

int proj_scratch_setup(int device)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return QKV_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device])
        return QKV_OK;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return QKV_ERR_HIP;
    g_scratch_ptr[device] = ptr;
    return QKV_OK;
}

}  // namespace qkv_detail

namespace {

void *scratch_ptr(int device)
{
    if (device < 0 || device >= kMaxScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

// run_proj and run_proj_noalloc: identical but for where the MFMA path's
// workspace lives (the handle's, grown with hipMalloc; or the static scratch)
int run_proj_impl(qkv_epilogue_t *h, const qkv_proj_args_t *pa, bool static_ws)
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
    const bool sep = pa->w_k || pa->w_v;            // three weight matrices instead of the concat one
    if (pa->w_format != QKV_WEIGHT_BF16 && pa->w_format != QKV_WEIGHT_E4M3)
        return fail(h, QKV_ERR_UNSUPPORTED, "unknown weight format %d", pa->w_format);
    const bool w8 = pa->w_format == QKV_WEIGHT_E4M3;
    const int64_t wel = w8 ? 1 : 2;                 // bytes per weight
    // the kernels address x and each weight matrix with 32-bit byte offsets
    if ((int64_t)a->nt * (pa->ld_x ? pa->ld_x : pa->hidden) * 2 > INT32_MAX ||
        (sep ? std::max(pl.nqt, pl.nkt) : N) * pa->hidden * wel > INT32_MAX)
        return fail(h, QKV_ERR_INVALID_ARG, "x and each weight matrix must span less than 2 GiB");
    if (sep && (!pa->w_k || !pa->w_v))
        return fail(h, QKV_ERR_INVALID_ARG, "w_k and w_v must be both NULL or both non-NULL");
    const int64_t ld_x = pa->ld_x ? pa->ld_x : pa->hidden;
    if (ld_x < pa->hidden || ld_x % 8 != 0)
        return fail(h, QKV_ERR_INVALID_ARG, "ld_x must be >= hidden and a multiple of 8");
    if (a->nt == 0)
        return QKV_OK;
    if (!pa->x || !pa->w || (uintptr_t)pa->x % 16 || (uintptr_t)pa->w % 16 || (uintptr_t)pa->w_k % 16 ||
        (uintptr_t)pa->w_v % 16)
        return fail(h, QKV_ERR_INVALID_ARG, "x and the weights must be non-NULL and 16-byte aligned");
    if (w8 && (!pa->w_scale || (uintptr_t)pa->w_scale % 4))
        return fail(h, QKV_ERR_INVALID_ARG, "E4M3 weights need w_scale (non-NULL, 4-byte aligned)");
    // the q, k, v weight sections: rows of the concat matrix, or three matrices
    const unsigned char *const w0 = static_cast<const unsigned char *>(pa->w);
    const unsigned char *const wsec[3] = {
        w0, sep ? static_cast<const unsigned char *>(pa->w_k) : w0 + pl.nqt * pa->hidden * wel,
        sep ? static_cast<const unsigned char *>(pa->w_v) : w0 + (pl.nqt + pl.nkt) * pa->hidden * wel};
    {
        // x and the weights are read while the outputs are written: no byte
        // in common (hull test on each range, conservative for strided rows)
        const int64_t nt = a->nt, cb = a->cache_dtype == QKV_CACHE_F16 ? 2 : 4;
        const int64_t cache_bytes = pl.n_slots * pl.n_ctx * pl.nkt * cb;
        const int64_t wrows[3] = {pl.nqt, pl.nkt, pl.nkt};
        uintptr_t ins[5][2] = {
            {(uintptr_t)pa->x, (uintptr_t)pa->x + (uintptr_t)(((nt - 1) * ld_x + pa->hidden) * 2)}};
        for (int s = 0; s < 3; ++s) {
            ins[1 + s][0] = (uintptr_t)wsec[s];
            ins[1 + s][1] = (uintptr_t)wsec[s] + (uintptr_t)(wrows[s] * pa->hidden * wel);
        }
        // the row scales (E4M3 only; else an empty range)
        ins[4][0] = (uintptr_t)pa->w_scale;
        ins[4][1] = w8 ? (uintptr_t)pa->w_scale + (uintptr_t)(N * 4) : (uintptr_t)pa->w_scale;
        const uintptr_t outs[5][2] = {
            {(uintptr_t)a->q, (uintptr_t)a->q + (uintptr_t)(((nt - 1) * pl.ld[0] + pl.nqt) * 4)},
            {(uintptr_t)a->k, (uintptr_t)a->k + (uintptr_t)(((nt - 1) * pl.ld[1] + pl.nkt) * 4)},
            {(uintptr_t)a->v, (uintptr_t)a->v + (uintptr_t)(((nt - 1) * pl.ld[2] + pl.nkt) * 4)},
            {(uintptr_t)a->kcache, (uintptr_t)a->kcache + (uintptr_t)cache_bytes},
            {(uintptr_t)a->vcache, (uintptr_t)a->vcache + (uintptr_t)cache_bytes}};
        const char *in_name[5] = {"x", sep ? "w" : "w (q rows)", sep ? "w_k" : "w (k rows)",
                                  sep ? "w_v" : "w (v rows)", "w_scale"};
        const char *out_name[5] = {"q", "k", "v", "kcache", "vcache"};
        for (int i = 0; i < 5; ++i)
            for (int o = 0; o < 5; ++o)
                if (ins[i][0] < outs[o][1] && outs[o][0] < ins[i][1])
                    return fail(h, QKV_ERR_ALIAS, "read-only %s overlaps output %s", in_name[i],
                                out_name[o]);
    }

    ProjParams pp;
    pp.x = static_cast<const uint16_t *>(pa->x);
    for (int s = 0; s < 3; ++s)
        pp.wsec[s] = reinterpret_cast<const uint16_t *>(wsec[s]);
    pp.sep = sep;
    pp.w8 = w8;
    pp.wscale = w8 ? pa->w_scale : nullptr;
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
    pp.rows = nullptr;
    pp.ksplit = 1;
    pp.part = nullptr;
    pp.device = h->device;
    pp.style = a->rope_style;

    // head_dim is 64 or 128 here: the short table holds every entry
    const InvTableSmall inv = small_table(handle_inv(h, a->theta, a->head_dim, a->freq_scale));
    hipStream_t st = (a->stream || a->use_stream) ? static_cast<hipStream_t>(a->stream) : h->stream;
    DeviceGuard g;
    hipError_t e = g.set(h->device);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "hipSetDevice(%d): %s", h->device, hipGetErrorString(e));
    MmPlan plan = {4, 4, 1, 1};
    if (pp.M > kGemvTok) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
        if (e != hipSuccess || cus <= 0)
            return fail(h, QKV_ERR_HIP, "compute-unit count: %s", hipGetErrorString(e));
        plan = mm_plan(pp.M, pp.N, pp.K, cus, pp.w8);
        pp.ksplit = plan.ksplit;
        {
            // the grid (tiles x splits) and the kernels' tile indices are 32-bit
            const int64_t bm = mm_bm(plan.mi, plan.wn), gt = plan.wn * plan.g;
            const int64_t blocks = ((pp.M + bm - 1) / bm) * ((pp.N / 64 + gt - 1) / gt) * pp.ksplit;
            if (blocks > INT32_MAX)
                return fail(h, QKV_ERR_UNSUPPORTED, "nt x q|k|v width too large (%lld tiles)",
                            (long long)blocks);
        }
        // The MFMA path's workspace (the handle's, grown on demand after the
        // device has finished with the old one): the launch's [nt][head_dim]
        // cos/sin table, the [nt] cache rows, and [ksplit][nt][N] partial sums
        // when k is split.
        const size_t tab = ((size_t)pp.M * (size_t)a->head_dim * sizeof(float) + 255) / 256 * 256;
        const size_t rows = ((size_t)pp.M * sizeof(int64_t) + 255) / 256 * 256;
        const size_t need =
            tab + rows + (pp.ksplit > 1 ? (size_t)pp.ksplit * pp.M * pp.N * sizeof(float) : 0);
        if (static_ws) {
            void *const sp = scratch_ptr(h->device);
            if (!sp)
                return fail(h, QKV_ERR_HIP, "the static workspace of device %d has no address "
                            "(handle creation could not look it up)", h->device);
            if (need > kScratchBytes)
                return fail(h, QKV_ERR_UNSUPPORTED,
                            "this call needs %zu bytes of workspace; the allocation-free entry point "
                            "has %zu (use qkv_epilogue_run_proj, or fewer tokens per call)",
                            need, kScratchBytes);
            char *ws = static_cast<char *>(sp);
            pp.rtab = reinterpret_cast<const float *>(ws);
            pp.rows = reinterpret_cast<const int64_t *>(ws + tab);
            pp.part = reinterpret_cast<float *>(ws + tab + rows);
        } else if (h->proj_ws_bytes < need) {
            // growing synchronizes the device and allocates: refused while the
            // stream is being captured, where neither is allowed
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            e = hipStreamIsCapturing(st, &cs);
            if (e != hipSuccess)
                return fail(h, QKV_ERR_HIP, "stream capture query: %s", hipGetErrorString(e));
            if (cs != hipStreamCaptureStatusNone)
                return fail(h, QKV_ERR_INVALID_ARG,
                            "this call needs %zu bytes of workspace and the handle holds %zu: make one call "
                            "of this size outside stream capture first",
                            need, h->proj_ws_bytes);
            e = hipDeviceSynchronize();
            if (e != hipSuccess)
                return fail(h, QKV_ERR_HIP, "device synchronize before growing the workspace: %s",
                            hipGetErrorString(e));
            if (h->proj_ws) {
                e = hipFree(h->proj_ws);
                h->proj_ws = nullptr;
                h->proj_ws_bytes = 0;
                if (e != hipSuccess)
                    return fail(h, QKV_ERR_HIP, "freeing the old workspace: %s", hipGetErrorString(e));
            }
            e = hipMalloc(&h->proj_ws, need);
            if (e != hipSuccess) {
                h->proj_ws = nullptr;
                return fail(h, QKV_ERR_HIP, "workspace of %zu bytes: %s", need, hipGetErrorString(e));
            }
            h->proj_ws_bytes = need;
        }
        if (!static_ws) {
            char *ws = static_cast<char *>(h->proj_ws);
            pp.rtab = reinterpret_cast<const float *>(ws);
            pp.rows = reinterpret_cast<const int64_t *>(ws + tab);
            pp.part = reinterpret_cast<float *>(ws + tab + rows);
        }
    }
    const bool f16 = a->cache_dtype == QKV_CACHE_F16;
    if (a->head_dim == 128)
        e = f16 ? launch_proj<true, 128>(pp, inv, st, plan) : launch_proj<false, 128>(pp, inv, st, plan);
    else
        e = f16 ? launch_proj<true, 64>(pp, inv, st, plan) : launch_proj<false, 64>(pp, inv, st, plan);
    if (e != hipSuccess)
        return fail(h, QKV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return QKV_OK;
}

}  // namespace

extern "C" int qkv_epilogue_run_proj(qkv_epilogue_t *h, const qkv_proj_args_t *pa)
{
    return run_proj_impl(h, pa, false);
}

extern "C" int qkv_epilogue_run_proj_noalloc(qkv_epilogue_t *h, const qkv_proj_args_t *pa)
{
    return run_proj_impl(h, pa, true);
}
