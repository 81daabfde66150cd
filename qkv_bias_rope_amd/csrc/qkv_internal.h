// qkv_internal.h -- internals shared by the HIP translation units of
// libqkv_epilogue.so (fused kernel, unfused chain, projection): vector slot
// types, the load/store policies and the handle.  Argument validation and
// planning are host-only and declared in qkv_plan.h.
// Not part of the public interface (that is include/qkv_epilogue.h).
#ifndef QKV_INTERNAL_H
#define QKV_INTERNAL_H

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "qkv_epilogue.h"
#include "qkv_plan.h"

namespace qkv_detail {

// Inverse-frequency table passed by value in the kernel arguments.
// The inverse-frequency table a launch passes by value in its kernel
// arguments.  HIP's host time for issuing a launch grows with the bytes of its
// arguments, so a launch whose head_dim/2 fits kSmallHalf (head_dim <= 128)
// passes only that many entries.
template <int N>
struct InvTableN {
    float v[N];
};
constexpr int kSmallHalf = 64;
using InvTable = InvTableN<kMaxHalf>;
using InvTableSmall = InvTableN<kSmallHalf>;

// The first kSmallHalf entries of a full table.
inline InvTableSmall small_table(const InvTable &t)
{
    InvTableSmall s;
    for (int i = 0; i < kSmallHalf; ++i)
        s.v[i] = t.v[i];
    return s;
}

template <int W>
struct alignas(4 * W) FVec {
    float e[W];
};

template <int W>
struct alignas(2 * W) HVec {
    _Float16 e[W];
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Plain load (biases, LDS).
template <int W>
__device__ __forceinline__ FVec<W> ld_vec(const float *p)
{
    return *reinterpret_cast<const FVec<W> *>(p);
}

// Load / store of q, k, v and the cache rows.  With STREAM (large launches,
// whose data is touched once and far exceeds the caches) they carry the
// nontemporal hint; small launches (decode) keep the default policy so data
// the producer just wrote, or the consumer reads next, stays cached.
template <int W, bool STREAM>
__device__ __forceinline__ FVec<W> ld_data(const float *p)
{
    if constexpr (!STREAM) {
        return ld_vec<W>(p);
    } else {
        FVec<W> r;
        if constexpr (W == 4) {
            const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
            r.e[0] = v.x;
            r.e[1] = v.y;
            r.e[2] = v.z;
            r.e[3] = v.w;
        } else {
            r.e[0] = __builtin_nontemporal_load(p);
        }
        return r;
    }
}

template <int W, bool STREAM>
__device__ __forceinline__ void st_data(float *p, const FVec<W> &v)
{
    if constexpr (!STREAM) {
        *reinterpret_cast<FVec<W> *>(p) = v;
    } else if constexpr (W == 4) {
        const f32x4 x = {v.e[0], v.e[1], v.e[2], v.e[3]};
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
    } else {
        __builtin_nontemporal_store(v.e[0], p);
    }
}

template <int W, bool F16, bool STREAM>
__device__ __forceinline__ void st_cache(void *cache, int64_t off, const FVec<W> &v)
{
    if constexpr (F16) {
        HVec<W> h;
#pragma unroll
        for (int e = 0; e < W; ++e)
            h.e[e] = static_cast<_Float16>(v.e[e]);  // v_cvt_f16_f32: RNE
        _Float16 *dst = static_cast<_Float16 *>(cache) + off;
        if constexpr (!STREAM) {
            *reinterpret_cast<HVec<W> *>(dst) = h;
        } else if constexpr (W == 4) {
            const f16x4 x = {h.e[0], h.e[1], h.e[2], h.e[3]};
            __builtin_nontemporal_store(x, reinterpret_cast<f16x4 *>(dst));
        } else {
            __builtin_nontemporal_store(h.e[0], dst);
        }
    } else {
        st_data<W, STREAM>(static_cast<float *>(cache) + off, v);
    }
}

// Stores that reach HBM while the kernel runs.  The L2 of each XCD is
// write-back: a plain (or merely non-temporal) store leaves its line dirty
// there, and the release at the end of the kernel writes every dirty line
// back after the last wave has finished -- a launch that writes a few MB per
// XCD pays for that writeback on its critical path.  A store at device scope
// (sc1) is written through the L2 as it is issued; with the non-temporal bit
// (nt) its line is also marked as streaming.  The global-store builtins carry
// only the nt bit, so these go through a raw buffer resource.  `base` should
// be the same for every lane of the wave (a section row, a cache row): the
// compiler loops over the distinct resources of a wave, once per value.
// q/k/v rows, read and written back in place, take both bits.  The K/V cache
// rows take the write-through bit alone: with the non-temporal bit as well
// the 4096-token 14B prefill measured 41.2-41.6 us against 40.0-40.4 (f16
// cache) and 44.5-44.8 against 41.9-42.1 (f32 cache) in same-process A/Bs;
// the 256-sequence batch was the same either way.
constexpr int kStreamStorePolicy = 2 /* nt */ | 16 /* sc1 */;
constexpr int kCacheStorePolicy = 16 /* sc1 */;

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *base)
{
    // raw buffer (stride 0); every offset below 2^31 bytes is in range; the
    // fourth word selects 32-bit data for untyped access
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}

// W floats at byte offset off from base
template <int W, int POL = kStreamStorePolicy>
__device__ __forceinline__ void st_stream(float *base, uint32_t off, const FVec<W> &v)
{
    const __amdgpu_buffer_rsrc_t r = stream_rsrc(base);
    if constexpr (W == 4) {
        const u32x4 u = {__builtin_bit_cast(unsigned, v.e[0]), __builtin_bit_cast(unsigned, v.e[1]),
                         __builtin_bit_cast(unsigned, v.e[2]), __builtin_bit_cast(unsigned, v.e[3])};
        __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, POL);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v.e[0]), r, (int)off, 0, POL);
    }
}

// W values converted to f16 (round to nearest even, per element) or kept f32,
// at element index idx of the cache row that starts at row_base
template <int W, bool F16>
__device__ __forceinline__ void st_stream_cache(void *row_base, uint32_t idx, const FVec<W> &v)
{
    if constexpr (F16) {
        const __amdgpu_buffer_rsrc_t r = stream_rsrc(row_base);
        HVec<W> h;
#pragma unroll
        for (int e = 0; e < W; ++e)
            h.e[e] = static_cast<_Float16>(v.e[e]);  // v_cvt_f16_f32: RNE
        if constexpr (W == 4) {
            const u32x2 u = __builtin_bit_cast(u32x2, h);
            __builtin_amdgcn_raw_buffer_store_b64(u, r, (int)(idx * 2u), 0, kCacheStorePolicy);
        } else {
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h.e[0]), r,
                                                  (int)(idx * 2u), 0, kCacheStorePolicy);
        }
    } else {
        st_stream<W, kCacheStorePolicy>(static_cast<float *>(row_base), idx * 4u, v);
    }
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


}  // namespace qkv_detail

struct qkv_epilogue {
    int device;
    int64_t n_ctx;
    hipStream_t stream;
    unsigned int *d_err;
    float inv_theta;
    int inv_hd;
    float inv_scale;
    qkv_detail::InvTable inv;
    char msg[512];
    // device workspace of the projection path (the long-prompt cos/sin
    // table), grown on demand, freed by destroy
    void *proj_ws;
    size_t proj_ws_bytes;
};

namespace qkv_detail {

int fail(qkv_epilogue *h, int code, const char *fmt, ...);

// Look up, once per device (that device current), the device address of the
// allocation-free projection's static workspace.  Called by create.
int proj_scratch_setup(int device);

// The handle's table for (theta, head_dim, freq_scale; 0 means 1), recomputed
// only when they change.
const InvTable &handle_inv(qkv_epilogue *h, float theta, int head_dim, float freq_scale);

}  // namespace qkv_detail

#endif  // QKV_INTERNAL_H
