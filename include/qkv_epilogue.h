/*
 * qkv_epilogue.h -- C ABI of the fused attention-input epilogue for MI355X
 * (gfx950).
 *
 * The operation (page "73 · D3-8 — G4 FusedQKV ported to CUDA", minfer CUDA
 * optimization steps, §2 and §3.2 Excerpt A): for every token t of a launch
 *
 *   1. add the biases:  q[t][j] += bq[j], k[t][j] += bk[j], v[t][j] += bv[j]
 *      (one f32 add each);
 *   2. rotate q and k with NeoX-paired rotary embedding: inside every head of
 *      head_dim elements, element i pairs with element i + head_dim/2 and the
 *      pair turns by the angle pos[t] * theta^(-2i/head_dim);
 *   3. write k and v back in place, and store them into the layer's KV cache
 *      at row pos[t] (page "07 · The allocator", §2.5: each per-layer region is
 *      n_ctx rows of n_kv_head*head_dim elements, the element of token t at
 *      dst[pos*nkt + j]), as f32 or as f16 rounded to nearest even.
 *
 * It is one kernel launch per call.  q, k and v are section base pointers, so
 * one concat q|k|v buffer and three separate buffers use the same entry point
 * (page 73, §2 "pointer-form").
 *
 * Numerics:
 *   - the inverse frequencies are the correctly rounded f32 of
 *     theta^(-2i/head_dim), computed once per (theta, head_dim) on the host in
 *     double precision;
 *   - the angle is the f32 product pos * inv[i];
 *   - cos and sin are evaluated in double precision and rounded to f32;
 *   - each rotated value is the f32 rounding of x0*c - x1*s (or x0*s + x1*c)
 *     evaluated in double (the products of two f32 values are exact there);
 *   - f16 cache values are IEEE binary16 round-to-nearest-even, subnormals
 *     kept, overflow to infinity.
 *
 * Conventions common to every call:
 *   - All tensor pointers are caller-owned DEVICE pointers on the handle's
 *     device.  The library never allocates, frees or copies tensor memory.
 *     The device memory it owns: each handle's 16-byte error word (create),
 *     each handle's projection workspace (grown by qkv_epilogue_run_proj,
 *     freed by destroy) and one static projection array per GPU
 *     (qkv_epilogue_run_proj_noalloc).
 *   - Calls that launch work are asynchronous on the given HIP stream and
 *     may be captured into a HIP graph.  Two calls block: qkv_epilogue_status
 *     (by design) and a qkv_epilogue_run_proj call that has to grow the
 *     handle's workspace (it synchronizes the device first; not allowed
 *     during capture).
 *   - Every function returns 0 on success or a negative QKV_ERR_* code; the
 *     text of the last failure is available from qkv_epilogue_last_error.
 *     There is no fallback path: an unsupported request is an error (page
 *     "06 · Assign + fusion", §2.1: a violated kernel invariant aborts rather
 *     than falling back).
 *   - A handle is not thread-safe: use one handle per host thread.  Launches
 *     of one handle on several streams may overlap, except the projection
 *     calls, which share the handle's workspace (or the GPU's static array):
 *     overlapping projection calls need separate handles (or, for the
 *     allocation-free entry point, ordering by the caller).
 */
#ifndef QKV_EPILOGUE_H
#define QKV_EPILOGUE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------- */
#define QKV_OK 0
#define QKV_ERR_INVALID_ARG   (-1) /* bad pointer, size, stride, dtype or theta */
#define QKV_ERR_ALIAS         (-2) /* output ranges overlap each other or an input */
#define QKV_ERR_UNSUPPORTED   (-3) /* a request outside what the kernels implement */
#define QKV_ERR_HIP           (-4) /* a HIP runtime call or launch failed */
#define QKV_ERR_POSITION_RANGE (-5) /* (status only) a pos/slot was out of range */

/* ---- cache element types ------------------------------------------------ */
#define QKV_CACHE_F32 0
#define QKV_CACHE_F16 1

/* ---- rotary styles ------------------------------------------------------ */
#define QKV_ROPE_NEOX 0         /* pair i with i + head_dim/2 (default) */
#define QKV_ROPE_INTERLEAVED 1  /* pair 2i with 2i+1 (GPT-J style) */

/* weight formats of qkv_epilogue_run_proj */
#define QKV_WEIGHT_BF16 0       /* bfloat16 weights (default) */
#define QKV_WEIGHT_E4M3 1       /* OCP 8-bit float E4M3 weights, one f32 scale per row */

/* Largest supported head_dim (the inverse-frequency table travels with the
 * launch and holds head_dim/2 values). */
#define QKV_MAX_HEAD_DIM 512

typedef struct qkv_epilogue qkv_epilogue_t;

typedef struct qkv_epilogue_config {
    int device;   /* HIP device ordinal the tensors live on */
    int64_t n_ctx;  /* positions per cache slot (rows of a one-sequence cache) */
    void *stream; /* hipStream_t used by qkv_epilogue_run; NULL = null stream */
} qkv_epilogue_config_t;

/*
 * Create a handle.  Allocates the handle and a 16-byte device error word on
 * cfg->device, and looks up the address of that device's static projection
 * array (the projection workspace itself is allocated later, by the first
 * qkv_epilogue_run_proj call that needs it).
 * Returns QKV_ERR_INVALID_ARG for a NULL out/cfg, n_ctx < 1 or a bad device
 * ordinal, QKV_ERR_HIP if the device cannot be used.  *out is NULL on error.
 */
int qkv_epilogue_create(qkv_epilogue_t **out, const qkv_epilogue_config_t *cfg);

/*
 * The epilogue over nt tokens of one layer, on the handle's stream.
 *
 *   q      [nt][n_head*head_dim]     f32, dense rows, biased + roped in place
 *   k      [nt][n_kv_head*head_dim]  f32, dense rows, biased + roped in place
 *   v      [nt][n_kv_head*head_dim]  f32, dense rows, biased in place
 *   bq     [n_head*head_dim]         f32 bias of q (read only)
 *   bk, bv [n_kv_head*head_dim]      f32 biases of k and v (read only)
 *   pos    [nt]                      int32 positions, read on the device
 *   kcache, vcache [n_ctx][n_kv_head*head_dim] of f32 (cache_dtype 0) or f16
 *          (cache_dtype 1): row pos[t] receives token t's k and v; no other
 *          row is touched.
 *   theta  rotary base (> 0, finite), e.g. 1e6.
 *
 * Dense rows only: for a concat q|k|v buffer with nt > 1 use
 * qkv_epilogue_run_ex and pass the concat row stride.  nt == 0 does nothing
 * and returns 0.  Equivalent to qkv_epilogue_run_ex with slot = NULL,
 * n_slots = 1, rope_style = NEOX, dense strides, the handle's n_ctx and
 * stream.
 *
 * A position outside [0, n_ctx) is reported by qkv_epilogue_status (that
 * token's q/k/v are still computed, its cache rows are not written); page
 * "07 · The allocator", §3.2 Excerpt 8: a position beyond the cache is a
 * hard error, never a silent overflow.
 */
int qkv_epilogue_run(qkv_epilogue_t *h, float *q, float *k, float *v,
                     const float *bq, const float *bk, const float *bv,
                     const int32_t *pos, void *kcache, void *vcache, int nt,
                     int n_head, int n_kv_head, int head_dim, float theta,
                     int cache_dtype);

typedef struct qkv_epilogue_args {
    float *q, *k, *v;               /* section bases (device) */
    const float *bq, *bk, *bv;      /* biases (device) */
    const int32_t *pos;             /* [nt] positions (device) */
    const int32_t *slot;            /* [nt] cache slot per token, or NULL = 0 */
    void *kcache, *vcache;          /* [n_slots][n_ctx][nkt] (device) */
    int64_t ld_q, ld_k, ld_v;       /* row strides in elements; 0 = dense */
    int64_t n_ctx;                  /* positions per slot; 0 = the handle's */
    int64_t n_slots;                /* slots in each cache; 0 = 1 */
    int nt, n_head, n_kv_head, head_dim;
    float theta;
    int cache_dtype;                /* QKV_CACHE_F32 / QKV_CACHE_F16 */
    int rope_style;                 /* QKV_ROPE_NEOX or QKV_ROPE_INTERLEAVED */
    void *stream;                   /* hipStream_t; NULL = the handle's */
    int use_stream;                 /* nonzero: launch on `stream` even if NULL */
    float freq_scale;               /* angle = pos * freq_scale * theta^(-2i/hd); 0 = 1 */
} qkv_epilogue_args_t;

/*
 * The general form.  Token t's cache row is slot[t]*n_ctx + pos[t] (slot 0
 * without a slot array); the multi-sequence reading of the page's single
 * region dst[pos*nkt + j].  Row strides let q, k and v be the sections of a
 * concat [nt][nqt + 2*nkt] buffer: q = base, k = base + nqt,
 * v = base + nqt + nkt, all with ld = nqt + 2*nkt.
 *
 * Errors (returned synchronously, nothing is launched):
 *   QKV_ERR_INVALID_ARG  NULL handle/args; a NULL tensor pointer when nt > 0;
 *                        nt < 0; n_head or n_kv_head < 1; head_dim <= 0, odd
 *                        or > QKV_MAX_HEAD_DIM; theta <= 0 or not finite; an
 *                        unknown cache_dtype; a stride below its row width;
 *                        n_ctx or n_slots < 0; a cache pointer not aligned to
 *                        its element size; 2^22 or more work units per
 *                        token (rows of about 2^25 elements) or more than
 *                        2^31-1 workgroups.
 *   QKV_ERR_ALIAS        two of q, k, v, kcache, vcache share an element, or
 *                        a read-only input (bias, pos, slot) overlaps one.
 *   QKV_ERR_UNSUPPORTED  rope_style is neither QKV_ROPE_NEOX nor
 *                        QKV_ROPE_INTERLEAVED (page "06 · Assign + fusion",
 *                        §3.2: a backend claims only the rotary styles its
 *                        kernel implements and rejects the others loudly).
 *
 * Rotary style and scale: with QKV_ROPE_INTERLEAVED pair i of a head is
 * (x[2i], x[2i+1]) instead of (x[i], x[i+head_dim/2]); freq_scale multiplies
 * every inverse frequency (the page's kernel takes freq_scale, §3.2 Excerpt
 * A): inv[i] = f32(freq_scale * theta^(-2i/head_dim)), the product taken in
 * double.  freq_scale must be finite and > 0 (0 means 1).
 *   QKV_ERR_HIP          the launch failed (text from the HIP runtime).
 * Duplicate cache rows within one call are a caller error: the row then holds
 * one of the colliding tokens' values.
 */
int qkv_epilogue_run_ex(qkv_epilogue_t *h, const qkv_epilogue_args_t *a);

/*
 * The q/k-norm variant (page "06 · Assign + fusion", §3.2: a per-head q/k norm
 * op and its fused form FusedQkvNorm, "the Qwen3 per-head-norm variant"; the
 * page gives no formula).  Per token: the biases that are given (bq, bk, bv
 * may each be NULL = no bias, as in the Qwen3 attention), then every q head
 * and every k head of head_dim values is scaled as
 *     y[j] = x[j] / sqrt(mean_j(x[j]^2) + eps) * w[j]
 * with w = w_q for q heads and w_k for k heads (both [head_dim] f32 device
 * arrays, shared by the heads of the section), then NeoX rotary embedding on q
 * and k, then the K/V row store -- as qkv_epilogue_run_ex otherwise.  v is
 * never normalised.  The sum of squares and the scaling are evaluated in
 * double and rounded once to f32.  One launch.
 *
 * Errors: those of qkv_epilogue_run_ex, plus QKV_ERR_INVALID_ARG for a NULL
 * or misaligned weight or eps < 0 / not finite, and QKV_ERR_ALIAS when a
 * weight overlaps an output.
 */
int qkv_epilogue_run_qk_norm(qkv_epilogue_t *h, const qkv_epilogue_args_t *a,
                             const float *w_q, const float *w_k, float eps);

/*
 * The projection that feeds the epilogue, with the epilogue in its output
 * stage (page "73 · D3-8 — G4 FusedQKV ported to CUDA", §2 and Excerpt C: one
 * matmul over the concat weight rows wq|wk|wv produces each token's q|k|v
 * row, which the epilogue consumes).  Per token t and output n:
 *     y[t][n] = sum_k x[t][k] * w[n][k]      (bf16 inputs, f32 accumulation)
 * then, on y split into its q, k, v sections, exactly the epilogue of
 * qkv_epilogue_run_ex: optional biases, rotary embedding of q and k in the
 * requested style (NeoX or interleaved) and frequency scale, the
 * sections written to epi.q / epi.k / epi.v (outputs only here) and the K/V
 * cache rows stored.  The GEMM runs on the matrix cores (MFMA) for more than
 * 4 tokens, as a weight-streaming GEMV for 1-4 tokens.  The epilogue runs on
 * the sums in registers, except when the batch has too few tiles to fill the
 * GPU: then the GEMM stores k-split partial sums and a second kernel adds
 * them in a fixed order and runs the epilogue (see Launches).
 *
 *   x   bf16 [nt][ld_x] activations (device, 16-byte aligned, ld_x % 8 == 0)
 *   w   bf16 [nqt + 2*nkt][hidden] concat weight rows q|k|v (device, aligned),
 *       or, with w_k and w_v given, the q weight [nqt][hidden] alone
 *   w_k, w_v  NULL (concat w), or the k and v weights [nkt][hidden] (device,
 *       aligned): the same page's layers whose q, k, v weights cannot share
 *       one concat matrix run three matmuls into one epilogue (§2); here the
 *       three matrices feed the one launch as they are, nothing repacked
 *   hidden  contraction length, a multiple of 64
 *   w_format  QKV_WEIGHT_BF16, or QKV_WEIGHT_E4M3: w (and w_k, w_v) then hold
 *       one byte per weight, an OCP 8-bit float in the E4M3 encoding (sign, 4
 *       exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7f/0xff NaN,
 *       no infinity), and row n of the q|k|v rows has the f32 scale
 *       w_scale[n]: y[t][n] = w_scale[n] * sum_k x[t][k] * w[n][k].  The same
 *       page's matmul runs on block-quantised weights; this is a weight-only
 *       8-bit form of it, which halves the bytes a decode step streams.
 *       E4M3 weights run on both kernels, at any token count: each E4M3
 *       value is converted to bf16 exactly and the products summed in f32 as
 *       for bf16 weights (the activations stay bf16: the matrix cores'
 *       8-bit forms take 8-bit floats on both sides), then multiplied by
 *       the scale (one more f32 rounding).
 *   w_scale  E4M3 only: f32 [nqt + 2*nkt] row scales (device, 4-byte
 *       aligned), indexed by the output's q|k|v column also when the weights
 *       come as three matrices; read-only, must not overlap an output.
 *
 * Limits (QKV_ERR_UNSUPPORTED otherwise): head_dim 64 or 128, q
 * and k/v widths multiples of 128; x and each weight matrix under 2 GiB
 * (QKV_ERR_INVALID_ARG).
 * The weights are read-only and may overlap one another, but none of x and
 * the weights may overlap an output or a cache (QKV_ERR_ALIAS); w_k and w_v
 * must be both NULL or both set (QKV_ERR_INVALID_ARG).
 *
 * Launches: 1-4 tokens run one weight-streaming kernel.  More tokens use a
 * workspace held by the handle: a cos/sin table of nt * head_dim * 4 bytes,
 * the tokens' cache rows (nt * 8 bytes) and, when k is split, the partial
 * sums (splits * nt * (nqt + 2*nkt) * 4 bytes, about 29 MB for 256 tokens of
 * the 14B shape); those launches are two kernels on the stream (the tables
 * and the GEMM, or the split GEMM and the summing epilogue).  A call that
 * needs more workspace than any before it synchronizes the device and
 * (re)allocates it: make that call outside graph capture (during capture it
 * returns QKV_ERR_INVALID_ARG and launches nothing).  All other calls
 * allocate nothing and never synchronize.  Calls on one handle share its
 * workspace: calls that may run concurrently (different streams) need
 * different handles.  The f32 sums are taken in a different order than a
 * plain loop: each output carries up to (hidden+2) * 2^-24 * sum_k |x w| of
 * accumulation error on top of the epilogue's own rounding.
 */
typedef struct qkv_proj_args {
    const void *x;          /* bf16 [nt][ld_x] */
    const void *w;          /* bf16 [nqt + 2*nkt][hidden], or [nqt][hidden] with w_k, w_v */
    int hidden;
    int64_t ld_x;           /* 0 = hidden */
    qkv_epilogue_args_t epi;  /* q/k/v are the outputs; biases may be NULL */
    const void *w_k;        /* NULL, or bf16 [nkt][hidden] */
    const void *w_v;        /* NULL, or bf16 [nkt][hidden] */
    int w_format;           /* QKV_WEIGHT_BF16 (0) or QKV_WEIGHT_E4M3 (1) */
    const float *w_scale;   /* E4M3: f32 [nqt + 2*nkt] row scales (device); else ignored */
} qkv_proj_args_t;

int qkv_epilogue_run_proj(qkv_epilogue_t *h, const qkv_proj_args_t *a);

/*
 * qkv_epilogue_run_proj for callers that cannot allocate device memory: code
 * being captured into a HIP graph, serving loops that must not call the
 * allocator, harnesses that forbid it.  Same arguments, results and errors as
 * qkv_epilogue_run_proj, and the same kernels; the launches of more than 4
 * tokens take their workspace (cos/sin table, cache rows, k-split partial
 * sums) from a static device array of 32 MiB (33554432 bytes) instead of the
 * handle's.  It never allocates, frees or synchronizes.
 *   - Limit: a call whose workspace exceeds 32 MiB returns
 *     QKV_ERR_UNSUPPORTED and launches nothing.  The workspace is nt *
 *     head_dim * 4 bytes plus nt * 8, each rounded up to 256, plus splits * nt
 *     * (nqt + 2*nkt) * 4 when the planner splits k (256 tokens of the 14B
 *     shape split four ways: 29.5 MB, within the limit; 4096 unsplit tokens:
 *     2.1 MB).  Use qkv_epilogue_run_proj beyond it.
 *   - The array exists once per GPU, for the life of the process; its
 *     address is looked up when a handle is created on that device
 *     (QKV_ERR_HIP here if that lookup failed).  Every call on one GPU, from
 *     any handle, uses the same array and leaves its contents behind: calls
 *     whose launches can overlap on one GPU (different streams, different
 *     threads) race on it and must be ordered by the caller.  Nothing in it
 *     needs clearing between calls: every element a launch reads was written
 *     earlier in the same call.
 */
int qkv_epilogue_run_proj_noalloc(qkv_epilogue_t *h, const qkv_proj_args_t *a);

/*
 * The same operation as qkv_epilogue_run_ex, computed by the UNFUSED chain the
 * fused kernel replaces: three bias-add launches (q, k, v), two rope launches
 * (q, k) and two store launches (K, V), seven kernels in that order (page "73 ·
 * D3-8 — G4 FusedQKV ported to CUDA", §1-§2: add_bias x3 + rope x2 +
 * store_kv x2 per layer).  Same arguments, validation, errors and numerics as
 * qkv_epilogue_run_ex (the rope launches evaluate cos/sin per pair instead of
 * once per token); results are bit-identical to the fused kernel.  For
 * same-binary A/B measurements of the fusion.
 */
int qkv_epilogue_run_unfused(qkv_epilogue_t *h, const qkv_epilogue_args_t *a);

/*
 * Blocking: synchronize the handle's device (every stream, so launches on any
 * stream and replays of captured graphs are all finished), then read and
 * clear the handle's device error word.  Returns QKV_ERR_POSITION_RANGE if
 * any token launched with this handle since the last status call had pos
 * outside [0, n_ctx) or slot outside [0, n_slots), QKV_ERR_HIP on a runtime
 * failure, else 0.  It also waits for unrelated work queued on the device.
 */
int qkv_epilogue_status(qkv_epilogue_t *h);

/* Text of the last non-zero return on this handle ("" if none).  The pointer
 * stays valid until the next call on the handle. */
const char *qkv_epilogue_last_error(const qkv_epilogue_t *h);

/* Free the handle, its error word and its projection workspace (no launch
 * of the handle may still be running).  NULL is a no-op. */
void qkv_epilogue_destroy(qkv_epilogue_t *h);

/* ---- host-only helpers (no device needed) ------------------------------- */

/*
 * The f32 inverse-frequency table the kernels use: out[i] = correctly rounded
 * theta^(-2i/head_dim), i < head_dim/2.  Returns QKV_ERR_INVALID_ARG for a
 * bad theta/head_dim or NULL out.
 */
int qkv_epilogue_inv_freq(float theta, int head_dim, float *out);

/* The same with a frequency scale: out[i] = f32(freq_scale * theta^(-2i/hd)),
 * the product in double (freq_scale finite and > 0). */
int qkv_epilogue_inv_freq_scaled(float theta, float freq_scale, int head_dim, float *out);

/*
 * Validate a request exactly as qkv_epilogue_run_ex does, without a handle
 * or a device.  n_ctx must be given (> 0) in *a.  Writes the reason to msg
 * (NUL-terminated, truncated to msg_len) and returns the code run_ex would.
 */
int qkv_epilogue_check_args(const qkv_epilogue_args_t *a, char *msg, size_t msg_len);

/*
 * The launch plan run_ex would use for *a (host-only): vector width of the
 * kernel variant (4 = 16-byte vector path, 1 = scalar path), work units per
 * token (a unit is two vector slots of one token's row), units per thread,
 * workgroup size, column blocks per token, tokens per workgroup, workgroup
 * count and dynamic LDS bytes.  Returns the check_args code.
 */
typedef struct qkv_epilogue_plan {
    int vec_width;
    int units_per_token;
    int units_per_thread;
    int block;
    int col_blocks;
    int tokens_per_block;
    int64_t grid;
    int lds_bytes;
} qkv_epilogue_plan_t;
int qkv_epilogue_plan(const qkv_epilogue_args_t *a, qkv_epilogue_plan_t *plan);

#ifdef __cplusplus
}
#endif
#endif /* QKV_EPILOGUE_H */
