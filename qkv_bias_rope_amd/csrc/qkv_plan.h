// qkv_plan.h -- host-only internals of libqkv_epilogue.so: the launch plan,
// argument validation and the inverse-frequency table (defined in
// qkv_host.cpp).  No HIP dependency: qkv_host.cpp also builds with a plain
// host compiler, for the sanitizer build of the tests.
// Not part of the public interface (that is include/qkv_epilogue.h).
#ifndef QKV_PLAN_H
#define QKV_PLAN_H

#include <cstddef>
#include <cstdint>

#include "qkv_epilogue.h"

namespace qkv_detail {

constexpr int kMaxHalf = QKV_MAX_HEAD_DIM / 2;
constexpr int kMaxBlock = 1024;

// LDS layout: int64 row[tb] | float cos[tb*half] | float sin[tb*half]
// (constexpr: callable from device code as well)
constexpr int lds_row_bytes(int tb)
{
    return ((tb * 8) + 15) & ~15;
}

struct Plan {
    int W;        // vector width: 4 (16-byte slots) or 1 (scalar slots)
    int U;        // units per token
    int nthr;     // threads per workgroup (one unit each)
    int ncb;      // column blocks per token
    int tb;       // tokens per workgroup (the planner uses 1)
    bool stream;  // nontemporal hints on the data
    bool norm;    // q/k-norm variant (column blocks hold whole heads)
    int style;    // QKV_ROPE_NEOX or QKV_ROPE_INTERLEAVED
    int64_t grid;
    int lds;
    int half;
    int64_t nqt, nkt;
    int64_t ld[3];
    int64_t n_ctx, n_slots;
};

int ceil_div(int64_t a, int64_t b);
void set_msg(char *msg, size_t len, const char *fmt, ...);

// check_and_plan flags
constexpr unsigned kPlanBiasOptional = 1u;  // NULL biases mean "no bias"
constexpr unsigned kPlanNorm = 2u;          // plan the q/k-norm variant

// Validate a request (the checks run_ex documents) and plan the fused launch.
// With kPlanNorm, wq/wk are the [head_dim] norm weights (checked for NULL,
// alignment and overlap with the outputs) and eps the norm epsilon.
int check_and_plan(const qkv_epilogue_args_t *a, int64_t n_ctx_default, Plan *pl, char *msg,
                   size_t mlen, unsigned flags = 0, const float *wq = nullptr,
                   const float *wk = nullptr, float eps = 0.0f);

// inv[i] = f32(freq_scale * theta^(-2i/head_dim)), computed in double and
// rounded once.
void host_inv_freq(float theta, int head_dim, float freq_scale, float *out);

}  // namespace qkv_detail

#endif  // QKV_PLAN_H
