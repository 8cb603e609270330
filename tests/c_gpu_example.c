/* A plain C consumer of librar.so on the GPU: allocates with the HIP runtime,
 * runs rar_allreduce_sgd through the C ABI, and checks the result bit for bit.
 * Integer-valued gradients keep every partial sum exact, so the expected mean
 * is the correctly rounded S/N in any order and the expected weights follow
 * from two binary32 roundings; both are computed here independently.
 * It runs twice: on separately allocated ranks, and on ranks carved from one
 * pool at the stride rar_rank_stride_tune picks.
 * Built by __graft_entry__.build() (gcc, C99); run by tests/test_gpu_parity.py.
 * Exit status 0: all ranks and the weights match. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rar.h"

#define N 6
#define P 100003

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
            return 2;                                                           \
        }                                                                       \
    } while (0)

int main(void)
{
    static float g[N][P], out[P], w[P], wout[P];
    static float mean[P], wexp[P];
    const float lr = 0.25f;
    for (int n = 0; n < N; ++n)
        for (int e = 0; e < P; ++e)
            g[n][e] = (float)((e * 7919 + n * 104729) % 2001 - 1000);  /* integers in [-1000, 1000] */
    for (int e = 0; e < P; ++e) {
        double s = 0.0;
        for (int n = 0; n < N; ++n)
            s += g[n][e];
        mean[e] = (float)(s / N);  /* double quotient, one rounding to binary32 */
        w[e] = (float)((e % 97) - 48) * 0.125f;
        volatile float step = lr * mean[e];  /* fl(lr * m), kept apart from the subtraction */
        wexp[e] = w[e] - step;
    }

    void *d[N];
    float *dw;
    for (int n = 0; n < N; ++n) {
        HIP_OK(hipMalloc(&d[n], sizeof(float) * P));
        HIP_OK(hipMemcpy(d[n], g[n], sizeof(float) * P, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc((void **)&dw, sizeof(float) * P));
    HIP_OK(hipMemcpy(dw, w, sizeof(float) * P, hipMemcpyHostToDevice));

    rar_plan_t plan = NULL;
    rar_status rc = rar_plan(N, P, RAR_F32, RAR_CHUNK_BALANCED, &plan);
    if (rc != RAR_OK) {
        fprintf(stderr, "rar_plan: %s\n", rar_strerror(rc));
        return 3;
    }
    rc = rar_allreduce_sgd(plan, d, dw, lr, P, NULL);
    if (rc != RAR_OK) {
        fprintf(stderr, "rar_allreduce_sgd: %s\n", rar_strerror(rc));
        return 3;
    }
    /* an argument error is reported before anything is enqueued */
    if (rar_allreduce_sgd(plan, d, dw, lr, P + 1, NULL) != RAR_EMISMATCH)
        return 4;
    HIP_OK(hipDeviceSynchronize());

    int bad = 0;
    for (int n = 0; n < N; ++n) {
        HIP_OK(hipMemcpy(out, d[n], sizeof(float) * P, hipMemcpyDeviceToHost));
        if (memcmp(out, mean, sizeof(float) * P) != 0) {
            fprintf(stderr, "rank %d differs from the exact mean\n", n);
            bad = 1;
        }
    }
    HIP_OK(hipMemcpy(wout, dw, sizeof(float) * P, hipMemcpyDeviceToHost));
    if (memcmp(wout, wexp, sizeof(float) * P) != 0) {
        fprintf(stderr, "weights differ\n");
        bad = 1;
    }
    /* the same ranks carved from one pool at the stride the library measures
     * fastest among four candidates, and reduced again */
    const int64_t MiB = (int64_t)1 << 20, s0 = 2 * MiB;  /* 400,012 bytes round up to 2 MiB */
    const int64_t pool_bytes = (N - 1) * (s0 + 3 * 2 * MiB) + (int64_t)sizeof(float) * P;
    char *pool;
    int64_t stride = 0;
    HIP_OK(hipMalloc((void **)&pool, (size_t)pool_bytes));
    rc = rar_rank_stride_tune(N, P, RAR_F32, pool, pool_bytes, 4, NULL, &stride);
    if (rc != RAR_OK || stride < s0 || stride > s0 + 3 * 2 * MiB || stride % (2 * MiB) != 0) {
        fprintf(stderr, "rar_rank_stride_tune: %s, stride %lld\n", rar_strerror(rc), (long long)stride);
        return 5;
    }
    void *pd[N];
    for (int n = 0; n < N; ++n) {
        pd[n] = pool + n * stride;
        HIP_OK(hipMemcpy(pd[n], g[n], sizeof(float) * P, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMemcpy(dw, w, sizeof(float) * P, hipMemcpyHostToDevice));
    if (rar_allreduce_sgd(plan, pd, dw, lr, P, NULL) != RAR_OK)
        return 3;
    HIP_OK(hipDeviceSynchronize());
    for (int n = 0; n < N; ++n) {
        HIP_OK(hipMemcpy(out, pd[n], sizeof(float) * P, hipMemcpyDeviceToHost));
        if (memcmp(out, mean, sizeof(float) * P) != 0) {
            fprintf(stderr, "pooled rank %d differs from the exact mean\n", n);
            bad = 1;
        }
    }
    HIP_OK(hipMemcpy(wout, dw, sizeof(float) * P, hipMemcpyDeviceToHost));
    if (memcmp(wout, wexp, sizeof(float) * P) != 0) {
        fprintf(stderr, "weights differ (pooled ranks)\n");
        bad = 1;
    }

    rar_plan_destroy(plan);
    for (int n = 0; n < N; ++n)
        HIP_OK(hipFree(d[n]));
    HIP_OK(hipFree(dw));
    HIP_OK(hipFree(pool));
    if (!bad)
        printf("c example ok: %d ranks x %d elements, bit-exact (separate buffers, and pooled at a %lld MiB stride)\n",
               N, P, (long long)(stride / MiB));
    return bad;
}
