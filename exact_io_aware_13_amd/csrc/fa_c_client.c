/*
 * fa_c_client.c -- a plain C consumer of the C ABI in include/fa.h.
 *
 * It shows the library in use without Python or PyTorch: device buffers from
 * hipMalloc, one stream, the forward on a causal problem through fa_fwd and
 * through fa_fwd_split with a caller workspace, the backward through fa_bwd,
 * and two calls that must be rejected before any work is enqueued.
 *
 * Inputs are bf16 values of a fixed integer hash (below), so that a checker
 * can rebuild them bit for bit.  The program writes, to the file named by its
 * one argument, the raw bits of: o and lse from fa_fwd, o and lse from
 * fa_fwd_split, then dq, dk, dv from fa_bwd (upstream gradient: the same hash
 * with another seed).  Exit status 0 means every call returned what it must.
 *
 *   usage: fa_c_client OUT.bin
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

enum { B = 1, H = 2, T = 300, D = 64 };

/* Value i of input stream `seed`: an integer hash mapped to [-2, 2), then
 * rounded to bf16 (round to nearest, ties to even). */
static uint16_t input_bits(uint32_t i, uint32_t seed) {
    uint32_t x = i * 2654435761u + seed * 40503u + 12345u;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    const float f = (float)(x >> 8) / 16777216.0f * 4.0f - 2.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            return 1;                                                             \
        }                                                                         \
    } while (0)

#define FA_EXPECT(call, want)                                                     \
    do {                                                                          \
        fa_status s_ = (call);                                                    \
        if (s_ != (want)) {                                                       \
            fprintf(stderr, "%s returned %d (%s), expected %d\n", #call, (int)s_,  \
                    fa_status_string(s_), (int)(want));                           \
            return 1;                                                             \
        }                                                                         \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT.bin\n", argv[0]);
        return 2;
    }
    const size_t n = (size_t)B * H * T * D, rows = (size_t)B * H * T;
    const float scale = 0.125f;
    uint16_t* host = malloc(n * 2);
    float* host_lse = malloc(rows * 4);
    if (!host || !host_lse) return 1;

    void *q, *k, *v, *o, *o2, *dout, *dq, *dk, *dv, *ws, *bws;
    float *lse, *lse2;
    HIP_OK(hipMalloc(&q, n * 2));
    HIP_OK(hipMalloc(&k, n * 2));
    HIP_OK(hipMalloc(&v, n * 2));
    HIP_OK(hipMalloc(&o, n * 2));
    HIP_OK(hipMalloc(&o2, n * 2));
    HIP_OK(hipMalloc(&dout, n * 2));
    HIP_OK(hipMalloc(&dq, n * 2));
    HIP_OK(hipMalloc(&dk, n * 2));
    HIP_OK(hipMalloc(&dv, n * 2));
    HIP_OK(hipMalloc((void**)&lse, rows * 4));
    HIP_OK(hipMalloc((void**)&lse2, rows * 4));
    void* ins[4] = {q, k, v, dout};
    for (uint32_t t = 0; t < 4; ++t) {
        for (size_t i = 0; i < n; ++i) host[i] = input_bits((uint32_t)i, t + 1);
        HIP_OK(hipMemcpy(ins[t], host, n * 2, hipMemcpyHostToDevice));
    }
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    /* Rejected before any work: a head size the library does not build, and
     * a causal split with more query rows than keys. */
    FA_EXPECT(fa_fwd(q, k, v, o, lse, B, H, T, 96, 1, scale, stream), FA_ERR_HEAD_DIM);
    FA_EXPECT(fa_fwd_split(q, k, v, o, lse, B, H, H, T, T - 1, D, 1, scale, 2, NULL, 0, stream), FA_ERR_SHAPE);

    FA_EXPECT(fa_fwd(q, k, v, o, lse, B, H, T, D, 1, scale, stream), FA_OK);

    const int64_t n_split = 3;
    const size_t ws_bytes = fa_fwd_split_workspace_bytes(B, H, T, T, D, n_split);
    if (ws_bytes == 0) {
        fprintf(stderr, "fa_fwd_split_workspace_bytes returned 0\n");
        return 1;
    }
    HIP_OK(hipMalloc(&ws, ws_bytes));
    FA_EXPECT(fa_fwd_split(q, k, v, o2, lse2, B, H, H, T, T, D, 1, scale, n_split, ws, ws_bytes, stream), FA_OK);

    const size_t bws_bytes = fa_bwd_workspace_bytes(B, H, T);
    HIP_OK(hipMalloc(&bws, bws_bytes > 0 ? bws_bytes : 16));
    FA_EXPECT(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, T, T, D, 1, scale, bws, bws_bytes, stream), FA_OK);
    HIP_OK(hipStreamSynchronize(stream));

    FILE* f = fopen(argv[1], "wb");
    if (!f) {
        perror(argv[1]);
        return 1;
    }
    void* os[2] = {o, o2};
    float* lses[2] = {lse, lse2};
    for (int r = 0; r < 2; ++r) {
        HIP_OK(hipMemcpy(host, os[r], n * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(host_lse, lses[r], rows * 4, hipMemcpyDeviceToHost));
        if (fwrite(host, 2, n, f) != n || fwrite(host_lse, 4, rows, f) != rows) return 1;
    }
    void* grads[3] = {dq, dk, dv};
    for (int g = 0; g < 3; ++g) {
        HIP_OK(hipMemcpy(host, grads[g], n * 2, hipMemcpyDeviceToHost));
        if (fwrite(host, 2, n, f) != n) return 1;
    }
    fclose(f);

    void* bufs[13] = {q, k, v, o, o2, dout, dq, dk, dv, lse, lse2, ws, bws};
    for (int i = 0; i < 13; ++i) HIP_OK(hipFree(bufs[i]));
    HIP_OK(hipStreamDestroy(stream));
    free(host);
    free(host_lse);
    printf("fa_c_client: %s (B=%d H=%d T=%d d=%d causal, scale %g): fa_fwd, fa_fwd_split (%lld splits), fa_bwd OK\n",
           argv[1], B, H, T, D, (double)scale, (long long)n_split);
    return 0;
}
