// hbm_probe.hip -- reference kernels that set the floor and the ceilings the
// epilogue's timings are read against on the same device (libqkv_probe.so,
// loaded by the benchmark only; the epilogue library does not contain them).
//
//  * empty:  a kernel that does nothing -- the per-launch floor of a grid of
//            a given size (dispatch, wave launch, end-of-kernel).
//  * empty_args: the same with 1280 bytes of kernel arguments, about what an
//            epilogue launch passes (its parameters and the 1 KB
//            inverse-frequency table): HIP's host path for a launch that
//            carries arguments.
//  * copy:   dst = src over 16-byte vectors, each thread issuing all its
//            loads before its stores.
//  * add:    buf += 1 in place over 16-byte vectors (the read/write mix of an
//            in-place elementwise pass).
//  * read:   a pass that only reads: every thread sums its 16-byte vectors
//            and each wave writes one float of the sum (4 bytes per 1 KB
//            times the vectors per thread), the traffic of a kernel that
//            streams a weight matrix once.
//  * rows:   the byte pattern of a batched decode step without any of its
//            arithmetic beyond one add: every element of a [nt][width] f32
//            matrix gets b[col] added in place, and the columns
//            [kv_col, kv_col + 2*nkt) of each row are also stored (f32, or
//            f16 rounded to nearest even) into row slot*n_ctx + pos of two
//            caches, the first nkt columns into kc and the next nkt into vc.
//            It reads and writes the same bytes as the epilogue on the same
//            launch: the matrix, the bias vector, pos/slot and the scattered
//            cache rows.
//
// Memory policy (argument `policy`):
//   0  plain loads and stores;
//   1  non-temporal loads and stores (the nt bit);
//   2  non-temporal loads, stores non-temporal at device scope (nt sc1),
//      which are written through the XCD's L2 as they are issued instead of
//      being written back by the end-of-kernel release;
//   3  non-temporal loads, stores at device scope without the non-temporal
//      bit (sc1); in the row pass only the cache rows take these stores and
//      the rows keep policy 2's (the epilogue's combination).
// Policy 2 stores go through a raw buffer resource whose base is the same
// for a whole workgroup (a block of the buffer, or a row), with offsets
// below 2^31.
//
// Every entry point checks its sizes and launch shape, launches on the given
// stream and returns 0, -1 for a rejected argument, or the HIP error code
// negated; nothing synchronizes.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNtDevice = 2 /* nt */ | 16 /* sc1 */;
constexpr int kDevice = 16 /* sc1 */;

__global__ void empty_kernel() {}

// kernel arguments of the size an epilogue launch passes (unused: the
// argument segment keeps its size, and the host copies every byte of it)
struct ArgBlock {
    float v[320];
};
__global__ void empty_args_kernel(ArgBlock) {}

template <int POL, typename T>
__device__ __forceinline__ T ld(const T *p)
{
    if constexpr (POL == 0)
        return *p;
    else
        return __builtin_nontemporal_load(p);
}

// 16 bytes at byte offset off from base (base shared by the workgroup)
template <int POL>
__device__ __forceinline__ void st16(void *base, uint32_t off, f32x4 v)
{
    f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<char *>(base) + off);
    if constexpr (POL == 0) {
        *p = v;
    } else if constexpr (POL == 1) {
        __builtin_nontemporal_store(v, p);
    } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0,
                                               POL == 3 ? kDevice : kNtDevice);
    }
}

template <int POL>
__device__ __forceinline__ void st8(void *base, uint32_t off, f16x4 v)
{
    f16x4 *p = reinterpret_cast<f16x4 *>(static_cast<char *>(base) + off);
    if constexpr (POL == 0) {
        *p = v;
    } else if constexpr (POL == 1) {
        __builtin_nontemporal_store(v, p);
    } else {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0,
                                              POL == 3 ? kDevice : kNtDevice);
    }
}

// Workgroup g covers vectors [g*blockDim*VPT, (g+1)*blockDim*VPT); thread t
// handles vectors t, t + blockDim, ... of that range.
template <int VPT, int POL>
__global__ __launch_bounds__(1024) void copy_kernel(f32x4 *__restrict__ dst,
                                                    const f32x4 *__restrict__ src, int64_t n)
{
    const int64_t g0 = (int64_t)blockIdx.x * blockDim.x * VPT;
    f32x4 r[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        r[j] = ld<POL>(src + min(g0 + (int64_t)j * blockDim.x + threadIdx.x, n - 1));
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t k = (int64_t)j * blockDim.x + threadIdx.x;
        if (g0 + k < n)
            st16<POL>(dst + g0, (uint32_t)(k * 16), r[j]);
    }
}

template <int VPT, int POL>
__global__ __launch_bounds__(1024) void add_kernel(f32x4 *__restrict__ buf, int64_t n)
{
    const int64_t g0 = (int64_t)blockIdx.x * blockDim.x * VPT;
    f32x4 r[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        r[j] = ld<POL>(buf + min(g0 + (int64_t)j * blockDim.x + threadIdx.x, n - 1));
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t k = (int64_t)j * blockDim.x + threadIdx.x;
        if (g0 + k < n)
            st16<POL>(buf + g0, (uint32_t)(k * 16), r[j] + 1.0f);
    }
}

// Workgroup g reads vectors [g*blockDim*VPT, (g+1)*blockDim*VPT) as copy does
// and wave w of it writes the sum of its lanes' vectors to out[g*waves + w].
template <int VPT, int POL>
__global__ __launch_bounds__(1024) void read_kernel(const f32x4 *__restrict__ src, int64_t n,
                                                    float *__restrict__ out)
{
    const int64_t g0 = (int64_t)blockIdx.x * blockDim.x * VPT;
    f32x4 r[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        r[j] = ld<POL>(src + min(g0 + (int64_t)j * blockDim.x + threadIdx.x, n - 1));
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const bool in = g0 + (int64_t)j * blockDim.x + threadIdx.x < n;
        acc += in ? (r[j].x + r[j].y) + (r[j].z + r[j].w) : 0.0f;
    }
    for (int m = 32; m >= 1; m >>= 1)
        acc += __shfl_xor(acc, m, 64);
    if ((threadIdx.x & 63) == 0)
        out[(int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = acc;
}

// One thread per 16-byte vector of a row, TPB rows per workgroup row of the
// grid (blockIdx.y); blockIdx.x walks the column vectors.
template <int TPB, bool F16, int POL>
__global__ __launch_bounds__(1024) void rows_kernel(float *__restrict__ x, const float *__restrict__ b,
                                                    int64_t nt, int64_t width4, int64_t kv_col4,
                                                    int64_t nkt4, const int32_t *__restrict__ pos,
                                                    const int32_t *__restrict__ slot, int64_t n_ctx,
                                                    void *__restrict__ kc, void *__restrict__ vc)
{
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * TPB;
    const int64_t cc = min(c, width4 - 1);
    const f32x4 bv = reinterpret_cast<const f32x4 *>(b)[cc];
    int64_t row[TPB];
    f32x4 v[TPB];
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
        const int64_t t = min(t0 + j, nt - 1);
        row[j] = (slot ? (int64_t)slot[t] : 0) * n_ctx + (int64_t)pos[t];
        v[j] = ld<POL>(reinterpret_cast<const f32x4 *>(x) + t * width4 + cc);
    }
    if (c >= width4)
        return;
    const int64_t kvc = c - kv_col4;
    const bool to_cache = kvc >= 0 && kvc < 2 * nkt4;
    void *const cache = kvc < nkt4 ? kc : vc;
    const int64_t cc4 = kvc < nkt4 ? kvc : kvc - nkt4;
    constexpr int cvec = F16 ? 8 : 16;  // bytes of four cache elements
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
        if (t0 + j >= nt)
            break;
        const f32x4 r = v[j] + bv;
        st16<POL == 3 ? 2 : POL>(x + (t0 + j) * width4 * 4, (uint32_t)(c * 16), r);
        if (to_cache) {
            void *const crow = static_cast<char *>(cache) + row[j] * nkt4 * cvec;
            if constexpr (F16) {
                const f16x4 h = {(_Float16)r.x, (_Float16)r.y, (_Float16)r.z, (_Float16)r.w};
                st8<POL>(crow, (uint32_t)(cc4 * 8), h);
            } else {
                st16<POL>(crow, (uint32_t)(cc4 * 16), r);
            }
        }
    }
}

int rc_of(hipError_t e)
{
    return e == hipSuccess ? 0 : -(int)e;
}

bool bad_block(int block)
{
    return block < 64 || block > 1024 || (block % 64) != 0;
}

template <int VPT, int POL>
void launch_copy(long long g, int block, hipStream_t st, f32x4 *d, const f32x4 *s, long long n16)
{
    hipLaunchKernelGGL((copy_kernel<VPT, POL>), dim3((unsigned)g), dim3(block), 0, st, d, s, (int64_t)n16);
}

template <int VPT, int POL>
void launch_add(long long g, int block, hipStream_t st, f32x4 *p, long long n16)
{
    hipLaunchKernelGGL((add_kernel<VPT, POL>), dim3((unsigned)g), dim3(block), 0, st, p, (int64_t)n16);
}

template <int VPT, int POL>
void launch_read(long long g, int block, hipStream_t st, const f32x4 *s, long long n16, float *out)
{
    hipLaunchKernelGGL((read_kernel<VPT, POL>), dim3((unsigned)g), dim3(block), 0, st, s, (int64_t)n16,
                       out);
}

template <int POL>
bool dispatch_read(int vpt, long long g, int block, hipStream_t st, const f32x4 *s, long long n, float *out)
{
    switch (vpt) {
    case 1: launch_read<1, POL>(g, block, st, s, n, out); return true;
    case 2: launch_read<2, POL>(g, block, st, s, n, out); return true;
    case 4: launch_read<4, POL>(g, block, st, s, n, out); return true;
    case 8: launch_read<8, POL>(g, block, st, s, n, out); return true;
    default: return false;
    }
}

template <int POL>
bool dispatch_copy(int vpt, long long g, int block, hipStream_t st, f32x4 *d, const f32x4 *s, long long n)
{
    switch (vpt) {
    case 1: launch_copy<1, POL>(g, block, st, d, s, n); return true;
    case 2: launch_copy<2, POL>(g, block, st, d, s, n); return true;
    case 4: launch_copy<4, POL>(g, block, st, d, s, n); return true;
    case 8: launch_copy<8, POL>(g, block, st, d, s, n); return true;
    default: return false;
    }
}

template <int POL>
bool dispatch_add(int vpt, long long g, int block, hipStream_t st, f32x4 *p, long long n)
{
    switch (vpt) {
    case 1: launch_add<1, POL>(g, block, st, p, n); return true;
    case 2: launch_add<2, POL>(g, block, st, p, n); return true;
    case 4: launch_add<4, POL>(g, block, st, p, n); return true;
    case 8: launch_add<8, POL>(g, block, st, p, n); return true;
    default: return false;
    }
}

template <int TPB, bool F16, int POL>
void launch_rows(dim3 grid, int block, hipStream_t st, float *x, const float *b, long long nt,
                 long long w4, long long kv4, long long nkt4, const int32_t *pos, const int32_t *slot,
                 long long n_ctx, void *kc, void *vc)
{
    hipLaunchKernelGGL((rows_kernel<TPB, F16, POL>), grid, dim3(block), 0, st, x, b, (int64_t)nt,
                       (int64_t)w4, (int64_t)kv4, (int64_t)nkt4, pos, slot, (int64_t)n_ctx, kc, vc);
}

template <bool F16, int POL>
bool dispatch_rows(int tpb, dim3 grid, int block, hipStream_t st, float *x, const float *b, long long nt,
                   long long w4, long long kv4, long long nkt4, const int32_t *pos, const int32_t *slot,
                   long long n_ctx, void *kc, void *vc)
{
    switch (tpb) {
    case 1: launch_rows<1, F16, POL>(grid, block, st, x, b, nt, w4, kv4, nkt4, pos, slot, n_ctx, kc, vc); return true;
    case 2: launch_rows<2, F16, POL>(grid, block, st, x, b, nt, w4, kv4, nkt4, pos, slot, n_ctx, kc, vc); return true;
    case 4: launch_rows<4, F16, POL>(grid, block, st, x, b, nt, w4, kv4, nkt4, pos, slot, n_ctx, kc, vc); return true;
    default: return false;
    }
}

}  // namespace

extern "C" {

// Number of workgroups a copy/add launch of n16 vectors uses (block threads,
// vpt vectors per thread).
long long qkv_probe_grid(long long n16, int block, int vpt)
{
    const long long per = (long long)block * vpt;
    return (n16 + per - 1) / per;
}

int qkv_probe_empty(int grid, int block, hipStream_t st)
{
    if (grid < 1 || bad_block(block))
        return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, st);
    return rc_of(hipGetLastError());
}

int qkv_probe_empty_args(int grid, int block, hipStream_t st)
{
    if (grid < 1 || bad_block(block))
        return -1;
    ArgBlock a;
    for (int i = 0; i < 320; ++i)
        a.v[i] = (float)i;
    hipLaunchKernelGGL(empty_args_kernel, dim3(grid), dim3(block), 0, st, a);
    return rc_of(hipGetLastError());
}

// dst/src: n16 16-byte vectors each, 16-byte aligned, not overlapping;
// vpt in {1, 2, 4, 8}; policy in {0, 1, 2}.
int qkv_probe_copy(void *dst, const void *src, long long n16, int block, int vpt, int policy,
                   hipStream_t st)
{
    if (!dst || !src || n16 < 1 || bad_block(block) || policy < 0 || policy > 3)
        return -1;
    if (((uintptr_t)dst | (uintptr_t)src) & 15u)
        return -1;
    const long long g = qkv_probe_grid(n16, block, vpt);
    if (g > 0x7fffffffLL)
        return -1;
    auto *d = static_cast<f32x4 *>(dst);
    auto *s = static_cast<const f32x4 *>(src);
    const bool ok = policy == 0   ? dispatch_copy<0>(vpt, g, block, st, d, s, n16)
                    : policy == 1 ? dispatch_copy<1>(vpt, g, block, st, d, s, n16)
                    : policy == 2 ? dispatch_copy<2>(vpt, g, block, st, d, s, n16)
                                  : dispatch_copy<3>(vpt, g, block, st, d, s, n16);
    return ok ? rc_of(hipGetLastError()) : -1;
}

// src: n16 16-byte vectors, 16-byte aligned; out: at least
// qkv_probe_grid(n16, block, vpt) * block / 64 floats, the per-wave sums;
// policy 0 plain or 1 non-temporal loads.
int qkv_probe_read(const void *src, long long n16, float *out, int block, int vpt, int policy,
                   hipStream_t st)
{
    if (!src || !out || n16 < 1 || bad_block(block) || ((uintptr_t)src & 15u) || policy < 0 ||
        policy > 1)
        return -1;
    const long long g = qkv_probe_grid(n16, block, vpt);
    if (g > 0x7fffffffLL)
        return -1;
    auto *p = static_cast<const f32x4 *>(src);
    const bool ok = policy == 0 ? dispatch_read<0>(vpt, g, block, st, p, n16, out)
                                : dispatch_read<1>(vpt, g, block, st, p, n16, out);
    return ok ? rc_of(hipGetLastError()) : -1;
}

// buf: n16 16-byte vectors, 16-byte aligned; every float gets 1 added.
int qkv_probe_add(void *buf, long long n16, int block, int vpt, int policy, hipStream_t st)
{
    if (!buf || n16 < 1 || bad_block(block) || ((uintptr_t)buf & 15u) || policy < 0 || policy > 3)
        return -1;
    const long long g = qkv_probe_grid(n16, block, vpt);
    if (g > 0x7fffffffLL)
        return -1;
    auto *p = static_cast<f32x4 *>(buf);
    const bool ok = policy == 0   ? dispatch_add<0>(vpt, g, block, st, p, n16)
                    : policy == 1 ? dispatch_add<1>(vpt, g, block, st, p, n16)
                    : policy == 2 ? dispatch_add<2>(vpt, g, block, st, p, n16)
                                  : dispatch_add<3>(vpt, g, block, st, p, n16);
    return ok ? rc_of(hipGetLastError()) : -1;
}

// x: [nt][width] f32 (width % 4 == 0, 16-byte aligned, nt*width*4 < 2^31
// bytes per row block), b: [width] f32; pos/slot: [nt] int32 (slot may be
// NULL: slot 0); kc/vc: caches of rows of nkt elements, f32 (f16 = 0) or f16
// (f16 = 1), large enough for every slot*n_ctx + pos the caller passes (the
// caller's contract: rows are not checked on the device).  kv_col % 4 == 0,
// nkt % 4 == 0, kv_col + 2*nkt <= width.  tpb rows per workgroup (1, 2, 4).
int qkv_probe_rows(float *x, const float *b, long long nt, long long width, long long kv_col,
                   long long nkt, const int32_t *pos, const int32_t *slot, long long n_ctx,
                   void *kc, void *vc, int f16, int block, int tpb, int policy, hipStream_t st)
{
    if (!x || !b || !pos || !kc || !vc || nt < 1 || width < 4 || (width & 3) || (kv_col & 3) ||
        (nkt & 3) || nkt < 4 || kv_col < 0 || kv_col + 2 * nkt > width || n_ctx < 1 ||
        bad_block(block) || policy < 0 || policy > 3 || width * 4 >= 0x7fffffffLL)
        return -1;
    if (((uintptr_t)x | (uintptr_t)b | (uintptr_t)kc | (uintptr_t)vc) & 15u)
        return -1;
    const long long w4 = width / 4;
    const long long gx = (w4 + block - 1) / block;
    const long long gy = (nt + tpb - 1) / tpb;
    if (gx > 0x7fffffffLL || gy > 65535)
        return -1;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    bool ok;
    if (f16)
        ok = policy == 0   ? dispatch_rows<true, 0>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
             : policy == 1 ? dispatch_rows<true, 1>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
             : policy == 2 ? dispatch_rows<true, 2>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
                           : dispatch_rows<true, 3>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc);
    else
        ok = policy == 0   ? dispatch_rows<false, 0>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
             : policy == 1 ? dispatch_rows<false, 1>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
             : policy == 2 ? dispatch_rows<false, 2>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc)
                           : dispatch_rows<false, 3>(tpb, grid, block, st, x, b, nt, w4, kv_col / 4, nkt / 4, pos, slot, n_ctx, kc, vc);
    return ok ? rc_of(hipGetLastError()) : -1;
}

}  // extern "C"
