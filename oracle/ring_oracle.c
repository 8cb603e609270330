/*
 * ring_oracle.c -- plain, slow CPU oracle for the ring all-reduce-mean and
 * the synchronous SGD update that follows it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library under ring_all_reduce_amd/) never links, calls or falls
 * back to it, and the two share no code, headers or tables.
 *
 * Sources (short names used below):
 *   [Gibiansky]  "Bringing HPC Techniques to Deep Learning", A. Gibiansky
 *                (Baidu SVAIL), Korean translation at wonjae.kim.
 *   [TrainMGPU]  "[AI System] Training With Multiple GPUs" (hecess blog).
 *   [DDPpage]    "[PyTorch] GPU 분산 학습 1 - DP / DDP / FSDP 개념".
 *
 * What is simulated, literally and in the pages' order:
 *   1. The flat array of every rank is cut into N chunks ([Gibiansky]
 *      §Scatter-reduce, first paragraph and the figure on splitting the
 *      array).  How the cut falls when N does not divide P is not stated;
 *      three readings are offered (see oracle_partition).
 *   2. Scatter-reduce, N-1 steps.  At step s rank n sends chunk (n-s) mod N
 *      to rank n+1, which adds the received values into its own copy of that
 *      chunk ([Gibiansky] §Scatter-reduce: rank n first sends chunk n and
 *      receives chunk n-1, and afterwards forwards what it last received;
 *      see also its step-1 table for five GPUs).  Every message is copied out of the
 *      sender ("snapshot") before any receiver writes, which is what a send
 *      followed by a receive means.
 *   3. The mean: after step 2 rank n holds the complete sum of chunk
 *      (n+1) mod N; it divides by N there ([Gibiansky] §The communication
 *      problem: gradients are averaged; [TrainMGPU] §Training Process,
 *      step 2: the average gradient).  Division is IEEE binary32 division.
 *   4. SGD, at the same owner: w <- w - lr*mean, rounded after the product
 *      and after the difference ([Gibiansky] §The communication problem: the
 *      averaged gradient is applied to the weights; [TrainMGPU] §Training
 *      Process, step 3).
 *   5. All-gather, N-1 steps.  At step s rank n sends chunk (n+1-s) mod N to
 *      rank n+1, which overwrites its copy ([Gibiansky] §Allgather and its
 *      step-1 table).
 *   Afterwards every rank holds the same array ([Gibiansky] §Ring allreduce;
 *   [DDPpage] §DDP: every GPU ends with the identical gradient).
 *
 * bf16 variant: the pages fix no bf16 behaviour.  Each rank's bf16 values are
 * widened exactly to binary32 working copies, steps 2-5 run in binary32, and
 * the bf16 arrays finally receive the round-to-nearest-even narrowing of the
 * binary32 mean; the SGD update uses the binary32 mean.
 *
 * Parallelism: OpenMP only over the elements of one message, so the result
 * does not depend on the thread count.  Build with -ffp-contract=off and
 * without any fast-math option so that every + - * / is one IEEE operation.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -4
#define ORACLE_ESCHEDULE -10 /* a rank would read and write one chunk in one step */

#define ORACLE_BALANCED 0
#define ORACLE_CEIL 1
#define ORACLE_ALIGN16 2

#define OMP_MIN_ELEMS 32768

static int mod_n(int64_t x, int n)
{
    int64_t r = x % n;
    return (int)(r < 0 ? r + n : r);
}

/* ---------------------------------------------------------------------- */
/* Chunk partition.                                                        */
/* ---------------------------------------------------------------------- */

/*
 * Cut P elements into N contiguous chunks; off has N+1 entries and chunk c is
 * [off[c], off[c+1]).  [Gibiansky] §Scatter-reduce says only "N smaller
 * chunks"; §Allreduce communication cost counts K/N values per send.
 *   BALANCED: sizes differ by at most one, the larger ones first.
 *   CEIL:     every chunk has ceil(P/N) elements except the tail, which takes
 *             what remains (it may be short, and trailing chunks may be empty).
 *   ALIGN16:  like CEIL but the common size is rounded up to a whole number of
 *             16-byte groups of elem_bytes-sized elements.
 */
int oracle_partition(int N, int64_t P, int mode, int elem_bytes, int64_t *off)
{
    if (N < 1 || P < 0 || off == NULL)
        return ORACLE_EINVAL;
    if (mode == ORACLE_BALANCED) {
        int64_t q = P / N, r = P % N;
        for (int c = 0; c <= N; ++c)
            off[c] = (int64_t)c * q + (c < r ? c : r);
        return ORACLE_OK;
    }
    if (mode == ORACLE_CEIL || mode == ORACLE_ALIGN16) {
        int64_t L = (P + N - 1) / N;
        if (mode == ORACLE_ALIGN16) {
            if (elem_bytes <= 0 || 16 % elem_bytes != 0)
                return ORACLE_EINVAL;
            int64_t g = 16 / elem_bytes;
            L = (L + g - 1) / g * g;
        }
        for (int c = 0; c < N; ++c) {
            int64_t o = (int64_t)c * L;
            off[c] = o < P ? o : P;
        }
        off[N] = P;
        return ORACLE_OK;
    }
    return ORACLE_EINVAL;
}

/* ---------------------------------------------------------------------- */
/* The literal ring on binary32 rank buffers.                             */
/* ---------------------------------------------------------------------- */

static int check_layout(int N, const int64_t *off)
{
    if (N < 1 || N > 4096 || off == NULL || off[0] != 0)
        return ORACLE_EINVAL;
    for (int c = 0; c < N; ++c)
        if (off[c + 1] < off[c])
            return ORACLE_EINVAL;
    return ORACLE_OK;
}

static int64_t max_chunk(int N, const int64_t *off)
{
    int64_t m = 0;
    for (int c = 0; c < N; ++c)
        if (off[c + 1] - off[c] > m)
            m = off[c + 1] - off[c];
    return m;
}

/* One ring transfer phase.  add != 0: scatter-reduce, the receiver adds.
 * add == 0: all-gather, the receiver overwrites.  At step 0 rank n sends
 * chunk n + first_shift; every later step it sends the chunk it received in
 * the step before, which is one chunk further back. */
static int ring_phase(int N, const int64_t *off, float *const *buf, float *snap, int64_t maxlen,
                      int add, int first_shift, int steps, int64_t *sent, int64_t *recv,
                      int32_t **trace)
{
    for (int s = 0; s < steps; ++s) {
        /* invariant that allows all N transfers of a step to proceed at
         * once in place: what rank n sends and what it receives are two
         * different chunks. */
        for (int n = 0; n < N; ++n) {
            int out_c = mod_n((int64_t)n + first_shift - s, N);
            int in_c = mod_n((int64_t)n - 1 + first_shift - s, N);
            if (out_c == in_c)
                return ORACLE_ESCHEDULE;
        }
        /* send: every rank copies its outgoing chunk into a message. */
        for (int n = 0; n < N; ++n) {
            int c = mod_n((int64_t)n + first_shift - s, N);
            int64_t len = off[c + 1] - off[c];
            if (sent)
                sent[n] += len;
            if (trace && *trace) {
                (*trace)[0] = add ? 0 : 1; /* phase */
                (*trace)[1] = s;
                (*trace)[2] = n; /* sender; the receiver is n+1 */
                (*trace)[3] = c; /* chunk */
                *trace += 4;
            }
            if (buf)
                memcpy(snap + (int64_t)n * maxlen, buf[n] + off[c], (size_t)len * sizeof(float));
        }
        /* receive: rank n+1 takes rank n's message. */
        for (int n = 0; n < N; ++n) {
            int dst = (n + 1) % N;
            int c = mod_n((int64_t)n + first_shift - s, N);
            int64_t len = off[c + 1] - off[c];
            if (recv)
                recv[dst] += len;
            if (!buf)
                continue;
            float *d = buf[dst] + off[c];
            const float *m = snap + (int64_t)n * maxlen;
            if (add) {
#pragma omp parallel for schedule(static) if (len > OMP_MIN_ELEMS)
                for (int64_t i = 0; i < len; ++i)
                    d[i] = d[i] + m[i];
            } else {
#pragma omp parallel for schedule(static) if (len > OMP_MIN_ELEMS)
                for (int64_t i = 0; i < len; ++i)
                    d[i] = m[i];
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Ring all-reduce-mean (+ SGD when w != NULL) of N binary32 rank buffers laid
 * out per off[0..N].  buf may be NULL: then only the per-rank counters of
 * elements sent and received are tallied (schedule-only run).  sent/recv are
 * accumulated into (caller zeroes them) and may be NULL.
 *
 * sr_steps / ag_steps cut the run short for inspection of intermediate
 * states: with sr_steps < N-1 only that many scatter-reduce steps run (no
 * mean, no all-gather); with ag_steps < N-1 the all-gather stops early.  A
 * negative value means all N-1 steps.  trace, when not NULL, receives four
 * int32 per transfer in execution order: phase (0 scatter-reduce,
 * 1 all-gather), step, sender rank, chunk; it needs 8*N*(N-1) entries.
 */
int oracle_ring_f32_ex(int N, const int64_t *off, float *const *buf, float *w, float lr,
                       int64_t *sent, int64_t *recv, int sr_steps, int ag_steps, int32_t *trace)
{
    int rc = check_layout(N, off);
    if (rc)
        return rc;
    if (sr_steps < 0 || sr_steps > N - 1)
        sr_steps = N - 1;
    if (ag_steps < 0 || ag_steps > N - 1)
        ag_steps = N - 1;
    int64_t maxlen = max_chunk(N, off);
    float *snap = NULL;
    if (buf && N > 1) {
        snap = (float *)malloc((size_t)N * (size_t)(maxlen ? maxlen : 1) * sizeof(float));
        if (!snap)
            return ORACLE_ENOMEM;
    }
    int32_t *tp = trace;
    /* scatter-reduce: rank n first sends chunk n */
    rc = ring_phase(N, off, buf, snap, maxlen, 1, 0, sr_steps, sent, recv, &tp);
    if (rc == ORACLE_OK && sr_steps == N - 1) {
        if (buf) {
            /* mean, and SGD, at the owner: rank n now holds all of chunk n+1 */
            const float fN = (float)N;
            for (int n = 0; n < N; ++n) {
                int c = (n + 1) % N;
                int64_t o = off[c], len = off[c + 1] - off[c];
                float *d = buf[n] + o;
#pragma omp parallel for schedule(static) if (len > OMP_MIN_ELEMS)
                for (int64_t i = 0; i < len; ++i) {
                    float m = d[i] / fN;
                    d[i] = m;
                    if (w) {
                        float step = lr * m;
                        w[o + i] = w[o + i] - step;
                    }
                }
            }
        }
        /* all-gather: rank n first sends chunk n+1 */
        rc = ring_phase(N, off, buf, snap, maxlen, 0, 1, ag_steps, sent, recv, &tp);
    }
    free(snap);
    return rc;
}

int oracle_ring_f32(int N, const int64_t *off, float *const *buf, float *w, float lr,
                    int64_t *sent, int64_t *recv)
{
    return oracle_ring_f32_ex(N, off, buf, w, lr, sent, recv, -1, -1, NULL);
}

/* ---------------------------------------------------------------------- */
/* bfloat16 storage, binary32 arithmetic.                                 */
/* ---------------------------------------------------------------------- */

/* bfloat16 is the upper half of a binary32 pattern, so widening is exact. */
float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 value to the nearest bfloat16, ties to the even pattern
 * (IEEE 754 roundTiesToEven applied to an 8-bit significand).  A NaN keeps
 * its sign and leading payload bits and is forced quiet. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t dropped = u & 0xffffu;
    uint32_t kept = u >> 16;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u; /* a carry into the exponent is the correct rounding, up to infinity */
    return (uint16_t)kept;
}

void oracle_f32_to_bf16_array(const float *x, uint16_t *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = oracle_f32_to_bf16(x[i]);
}

void oracle_bf16_to_f32_array(const uint16_t *x, float *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = oracle_bf16_to_f32(x[i]);
}

/*
 * Ring all-reduce-mean (+ SGD) of N bfloat16 rank buffers.  in[n] and out[n]
 * may be the same array.  Every rank gets a binary32 working copy, the ring
 * runs on those, and out[n] receives the bf16 rounding of its final copy.
 */
int oracle_ring_bf16(int N, const int64_t *off, const uint16_t *const *in, uint16_t *const *out,
                     float *w, float lr, int64_t *sent, int64_t *recv)
{
    int rc = check_layout(N, off);
    if (rc)
        return rc;
    int64_t P = off[N];
    float **work = (float **)calloc((size_t)N, sizeof(float *));
    if (!work)
        return ORACLE_ENOMEM;
    for (int n = 0; n < N && rc == ORACLE_OK; ++n) {
        work[n] = (float *)malloc((size_t)(P ? P : 1) * sizeof(float));
        if (!work[n])
            rc = ORACLE_ENOMEM;
        else
            oracle_bf16_to_f32_array(in[n], work[n], P);
    }
    if (rc == ORACLE_OK)
        rc = oracle_ring_f32(N, off, work, w, lr, sent, recv);
    if (rc == ORACLE_OK)
        for (int n = 0; n < N; ++n)
            oracle_f32_to_bf16_array(work[n], out[n], P);
    for (int n = 0; n < N; ++n)
        free(work[n]);
    free(work);
    return rc;
}

/* ---------------------------------------------------------------------- */
/* Prior art: a single reducer (parameter server / master GPU).           */
/* ---------------------------------------------------------------------- */

/*
 * [Gibiansky] §The communication problem: every GPU sends its whole gradient
 * to one reducer GPU, which averages and sends the result back to all;
 * [TrainMGPU] §Training Process steps 2-4 and [DDPpage] §DP describe the same
 * shape.  Rank 0 is the reducer; it adds the arrivals in rank order
 * g0 + g1 + ... + g(N-1), divides by N, applies SGD and broadcasts.
 * buf may be NULL (counters only).
 */
int oracle_naive_f32(int N, int64_t P, float *const *buf, float *w, float lr, int64_t *sent,
                     int64_t *recv)
{
    if (N < 1 || P < 0)
        return ORACLE_EINVAL;
    for (int n = 1; n < N; ++n) {
        if (sent)
            sent[n] += P;
        if (recv)
            recv[0] += P;
    }
    if (buf) {
        float *acc = buf[0];
        const float fN = (float)N;
        for (int n = 1; n < N; ++n) {
            const float *g = buf[n];
#pragma omp parallel for schedule(static) if (P > OMP_MIN_ELEMS)
            for (int64_t i = 0; i < P; ++i)
                acc[i] = acc[i] + g[i];
        }
#pragma omp parallel for schedule(static) if (P > OMP_MIN_ELEMS)
        for (int64_t i = 0; i < P; ++i) {
            float m = acc[i] / fN;
            acc[i] = m;
            if (w) {
                float step = lr * m;
                w[i] = w[i] - step;
            }
        }
        for (int n = 1; n < N; ++n)
            memcpy(buf[n], acc, (size_t)P * sizeof(float));
    }
    for (int n = 1; n < N; ++n) {
        if (sent)
            sent[0] += P;
        if (recv)
            recv[n] += P;
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */

void oracle_set_threads(int t)
{
#ifdef _OPENMP
    if (t > 0)
        omp_set_num_threads(t);
#else
    (void)t;
#endif
}

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
