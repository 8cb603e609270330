/* Compiled as C99 against include/rar.h and linked with librar.so by
 * tests/test_abi_host.py: checks that the header is plain C and that the
 * host-only entry points behave as declared.  No device work. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rar.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

int main(void)
{
    rar_plan_t plan = NULL;
    CHECK(rar_plan(4, 1000003, RAR_F32, RAR_CHUNK_BALANCED, &plan) == RAR_OK && plan != NULL);
    int64_t off = -1, len = -1, sent = 0, recv = 0, total = 0;
    int owner = -1;
    for (int c = 0; c < 4; ++c) {
        CHECK(rar_plan_chunk(plan, c, &off, &len, &owner) == RAR_OK);
        CHECK(off == total && owner == (c + 3) % 4);
        CHECK(len == (c < 3 ? 250001 : 250000));
        total += len;
    }
    CHECK(total == 1000003);
    CHECK(rar_plan_chunk(plan, 4, &off, &len, &owner) == RAR_EINVAL);
    for (int n = 0; n < 4; ++n) {
        CHECK(rar_plan_traffic(plan, n, &sent, &recv) == RAR_OK);
        CHECK(sent > 0 && sent < 2 * 1000003 && recv > 0 && recv < 2 * 1000003);
    }
    /* argument checks come before any device work */
    void *bufs[4] = {NULL, NULL, NULL, NULL};
    CHECK(rar_allreduce_mean(plan, bufs, 1000003, NULL) == RAR_EINVAL);
    CHECK(rar_allreduce_mean(plan, bufs, 7, NULL) == RAR_EMISMATCH);
    CHECK(rar_plan_set_algo(plan, RAR_ALGO_RING) == RAR_OK);
    CHECK(rar_plan_set_grid(plan, -1) == RAR_EINVAL);
    CHECK(rar_plan_destroy(plan) == RAR_OK);
    CHECK(rar_plan(0, 10, RAR_F32, RAR_CHUNK_BALANCED, &plan) == RAR_EINVAL && plan == NULL);

    int64_t numel[3] = {10, 20, 30};
    rar_buckets_t b = NULL;
    int nb = 0;
    int64_t mx = 0;
    CHECK(rar_bucket_plan(3, numel, RAR_F32, 4 * 25, &b) == RAR_OK);
    CHECK(rar_bucket_count(b, &nb, &mx) == RAR_OK && nb == 3 && mx == 25);
    CHECK(rar_bucket_destroy(b) == RAR_OK);

    CHECK(strlen(rar_strerror(RAR_EALIGN)) > 0 && strlen(rar_strerror((rar_status)-77)) > 0);
    CHECK(rar_version() >= 100);
    printf("c abi ok\n");
    {
        int64_t stride = 0;
        CHECK(rar_rank_stride(300000000, RAR_F32, &stride) == RAR_OK);
        CHECK(stride == (int64_t)1146 << 20);
        CHECK(stride % ((int64_t)4 << 20) == ((int64_t)2 << 20));
        CHECK(rar_rank_stride(-1, RAR_F32, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride(10, RAR_BF16, NULL) == RAR_EINVAL);
        /* measured advice: every call below returns before any device work */
        void *fake = (void *)((uintptr_t)1 << 40), *odd = (void *)(((uintptr_t)1 << 40) + 8);
        const int64_t big = (int64_t)1 << 34, MiB = (int64_t)1 << 20;
        CHECK(rar_rank_stride_tune(1, 1000, RAR_F32, NULL, 0, 4, NULL, &stride) == RAR_OK && stride == 2 * MiB);
        CHECK(rar_rank_stride_tune(4, 0, RAR_F32, NULL, 0, 4, NULL, &stride) == RAR_OK && stride == 2 * MiB);
        CHECK(rar_rank_stride_tune(1, 300000000, RAR_F32, NULL, 0, 4, NULL, &stride) == RAR_OK && stride == 1146 * MiB);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, NULL, big, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, odd, big, 4, NULL, &stride) == RAR_EALIGN);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, fake, 6 * MiB, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, fake, big, 0, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, fake, big, RAR_MAX_STRIDE_CANDIDATES + 1, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(0, 1000, RAR_F32, fake, big, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(RAR_MAX_RANKS + 1, 1000, RAR_F32, fake, big, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, 1000, (rar_dtype)7, fake, big, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, -1, RAR_F32, fake, big, 4, NULL, &stride) == RAR_EINVAL);
        CHECK(rar_rank_stride_tune(4, 1000, RAR_F32, fake, big, 4, NULL, NULL) == RAR_EINVAL);
    }
    return 0;
}
