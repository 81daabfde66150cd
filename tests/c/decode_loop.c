/*
 * A decode step issued from C, with no Python in the process: one
 * qkv_epilogue_run_ex call per layer, each layer with its own q, k, v,
 * biases, position and f16 K/V caches (separate section buffers, one token),
 * all on one stream created here.  After `warmup` steps it times `steps`
 * steps with HIP events on that stream, and the host time spent issuing them
 * (the library's own host path: argument checks, planning and the launch),
 * then prints one JSON line.  The buffers are zero-filled: the values do not
 * change the work.
 *
 * usage: decode_loop n_head n_kv_head head_dim layers steps warmup
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <time.h>

#include "qkv_epilogue.h"

enum { Q, K, V, BQ, BK, BV, POS, KC, VC, NBUF };

static int fail(const char *what)
{
    fprintf(stderr, "decode_loop: %s\n", what);
    return 1;
}

static double now_us(void)
{
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return t.tv_sec * 1e6 + t.tv_nsec * 1e-3;
}

int main(int argc, char **argv)
{
    if (argc != 7)
        return fail("usage: decode_loop n_head n_kv_head head_dim layers steps warmup");
    const int n_head = atoi(argv[1]), n_kv_head = atoi(argv[2]), head_dim = atoi(argv[3]);
    const int layers = atoi(argv[4]), steps = atoi(argv[5]), warmup = atoi(argv[6]);
    if (n_head < 1 || n_kv_head < 1 || head_dim < 2 || layers < 1 || layers > 1024 || steps < 1 ||
        warmup < 0)
        return fail("bad arguments");
    const int64_t n_ctx = 4096;
    const size_t nqt = (size_t)n_head * head_dim, nkt = (size_t)n_kv_head * head_dim;
    const size_t bytes[NBUF] = {nqt * 4, nkt * 4, nkt * 4, nqt * 4, nkt * 4, nkt * 4, 4,
                                (size_t)n_ctx * nkt * 2, (size_t)n_ctx * nkt * 2};

    hipStream_t st;
    if (hipStreamCreate(&st) != hipSuccess)
        return fail("stream");
    qkv_epilogue_config_t cfg = {0, n_ctx, st};
    qkv_epilogue_t *h = NULL;
    if (qkv_epilogue_create(&h, &cfg) != QKV_OK)
        return fail("create");

    qkv_epilogue_args_t *args = calloc((size_t)layers, sizeof *args);
    void **dev = calloc((size_t)layers * NBUF, sizeof *dev);
    if (!args || !dev)
        return fail("host memory");
    for (int l = 0; l < layers; ++l) {
        void **d = dev + (size_t)l * NBUF;
        for (int i = 0; i < NBUF; ++i)
            if (hipMalloc(&d[i], bytes[i]) != hipSuccess || hipMemset(d[i], 0, bytes[i]) != hipSuccess)
                return fail("device buffer");
        const int32_t pos = 7 + l;
        if (hipMemcpy(d[POS], &pos, 4, hipMemcpyHostToDevice) != hipSuccess)
            return fail("position");
        qkv_epilogue_args_t *a = &args[l];
        a->q = (float *)d[Q];
        a->k = (float *)d[K];
        a->v = (float *)d[V];
        a->bq = (const float *)d[BQ];
        a->bk = (const float *)d[BK];
        a->bv = (const float *)d[BV];
        a->pos = (const int32_t *)d[POS];
        a->kcache = d[KC];
        a->vcache = d[VC];
        a->n_ctx = n_ctx;
        a->nt = 1;
        a->n_head = n_head;
        a->n_kv_head = n_kv_head;
        a->head_dim = head_dim;
        a->theta = 1.0e6f;
        a->cache_dtype = QKV_CACHE_F16;
        a->rope_style = QKV_ROPE_NEOX;
        a->stream = st;
        a->use_stream = 1;
    }
    if (hipDeviceSynchronize() != hipSuccess)
        return fail("set-up");

    int rc = 0;
    for (int s = 0; s < warmup; ++s)
        for (int l = 0; l < layers; ++l)
            rc |= qkv_epilogue_run_ex(h, &args[l]);
    if (rc != QKV_OK || hipStreamSynchronize(st) != hipSuccess)
        return fail("warm-up launches");

    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
        return fail("events");
    hipEventRecord(e0, st);
    const double t0 = now_us();
    for (int s = 0; s < steps; ++s)
        for (int l = 0; l < layers; ++l)
            rc |= qkv_epilogue_run_ex(h, &args[l]);
    const double t1 = now_us();
    hipEventRecord(e1, st);
    if (rc != QKV_OK || hipEventSynchronize(e1) != hipSuccess)
        return fail("timed launches");
    float ms = 0.0f;
    hipEventElapsedTime(&ms, e0, e1);
    if (qkv_epilogue_status(h) != QKV_OK)
        return fail(qkv_epilogue_last_error(h));
    const double calls = (double)steps * layers;
    printf("{\"us_per_layer\": %.4f, \"host_issue_us_per_call\": %.4f, \"layers\": %d, \"steps\": %d}\n",
           ms * 1e3 / calls, (t1 - t0) / calls, layers, steps);

    for (size_t i = 0; i < (size_t)layers * NBUF; ++i)
        hipFree(dev[i]);
    free(dev);
    free(args);
    qkv_epilogue_destroy(h);
    hipStreamDestroy(st);
    return 0;
}
