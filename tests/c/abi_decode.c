/*
 * A C consumer of libqkv_epilogue.so, with no Python in the process: one call
 * of qkv_epilogue_run (caller-owned device buffers, the handle's stream) on
 * inputs read from a file, the outputs written to another.  It links the
 * library and the HIP runtime only.  The GPU test that drives it writes the
 * inputs and checks the outputs against the oracle.
 *
 * Input file: int32 nt, n_head, n_kv_head, head_dim, n_ctx, cache_dtype;
 * float32 theta; then q, k, v, bq, bk, bv (float32), pos (int32), and the
 * K and V caches' initial contents (n_ctx rows of f32 or f16 elements).
 * Output file: q, k, v, then the two caches, in the same layouts.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "qkv_epilogue.h"

enum { Q, K, V, BQ, BK, BV, POS, KC, VC, NBUF };

static int fail(const char *what)
{
    fprintf(stderr, "abi_decode: %s\n", what);
    return 1;
}

int main(int argc, char **argv)
{
    if (argc != 3)
        return fail("usage: abi_decode IN OUT");
    FILE *in = fopen(argv[1], "rb");
    if (!in)
        return fail("cannot open the input file");
    int32_t hdr[6];
    float theta;
    if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&theta, sizeof theta, 1, in) != 1)
        return fail("short header");
    const int nt = hdr[0], n_head = hdr[1], n_kv_head = hdr[2], head_dim = hdr[3];
    const int64_t n_ctx = hdr[4];
    const int cache_dtype = hdr[5];
    const size_t nqt = (size_t)n_head * head_dim, nkt = (size_t)n_kv_head * head_dim;
    const size_t cb = cache_dtype == QKV_CACHE_F16 ? 2 : 4;
    const size_t bytes[NBUF] = {nt * nqt * 4, nt * nkt * 4, nt * nkt * 4, nqt * 4, nkt * 4, nkt * 4,
                                (size_t)nt * 4, (size_t)n_ctx * nkt * cb, (size_t)n_ctx * nkt * cb};
    void *host[NBUF], *dev[NBUF];
    for (int i = 0; i < NBUF; ++i) {
        host[i] = malloc(bytes[i]);
        if (!host[i] || fread(host[i], 1, bytes[i], in) != bytes[i])
            return fail("short input");
        if (hipMalloc(&dev[i], bytes[i]) != hipSuccess ||
            hipMemcpy(dev[i], host[i], bytes[i], hipMemcpyHostToDevice) != hipSuccess)
            return fail("device buffer");
    }
    fclose(in);

    qkv_epilogue_config_t cfg = {0, n_ctx, NULL};
    qkv_epilogue_t *h = NULL;
    if (qkv_epilogue_create(&h, &cfg) != QKV_OK)
        return fail("qkv_epilogue_create");
    int rc = qkv_epilogue_run(h, (float *)dev[Q], (float *)dev[K], (float *)dev[V], (const float *)dev[BQ],
                              (const float *)dev[BK], (const float *)dev[BV], (const int32_t *)dev[POS],
                              dev[KC], dev[VC], nt, n_head, n_kv_head, head_dim, theta, cache_dtype);
    if (rc != QKV_OK) {
        fprintf(stderr, "abi_decode: run returned %d: %s\n", rc, qkv_epilogue_last_error(h));
        return 1;
    }
    rc = qkv_epilogue_status(h);
    if (rc != QKV_OK) {
        fprintf(stderr, "abi_decode: status %d: %s\n", rc, qkv_epilogue_last_error(h));
        return 1;
    }
    qkv_epilogue_destroy(h);

    FILE *out = fopen(argv[2], "wb");
    if (!out)
        return fail("cannot open the output file");
    const int outs[5] = {Q, K, V, KC, VC};
    for (int j = 0; j < 5; ++j) {
        const int i = outs[j];
        if (hipMemcpy(host[i], dev[i], bytes[i], hipMemcpyDeviceToHost) != hipSuccess)
            return fail("copy back");
        if (fwrite(host[i], 1, bytes[i], out) != bytes[i])
            return fail("short output");
    }
    fclose(out);
    for (int i = 0; i < NBUF; ++i) {
        hipFree(dev[i]);
        free(host[i]);
    }
    return 0;
}
