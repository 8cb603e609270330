/* A plain C consumer of librar.so on the GPU: allocates with the HIP runtime,
 * runs rar_allreduce_sgd through the C ABI, and checks the result bit for bit.
 * Integer-valued gradients keep every partial sum exact, so the expected mean
 * is the correctly rounded S/N in any order and the expected weights follow
 * from two binary32 roundings; both are computed here independently.
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
    rar_plan_destroy(plan);
    for (int n = 0; n < N; ++n)
        HIP_OK(hipFree(d[n]));
    HIP_OK(hipFree(dw));
    if (!bad)
        printf("c example ok: %d ranks x %d elements, bit-exact\n", N, P);
    return bad;
}
