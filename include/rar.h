/*
 * rar.h -- C ABI of librar.so: ring all-reduce-mean and the synchronous SGD
 * update of data-parallel training, for N logical ranks whose gradient
 * buffers all sit in the HBM of one MI355X (gfx950).
 *
 * Sources (short names):
 *   [Gibiansky]  "Bringing HPC Techniques to Deep Learning", A. Gibiansky,
 *                Baidu SVAIL (Korean translation at wonjae.kim).
 *   [TrainMGPU]  "[AI System] Training With Multiple GPUs".
 *   [DDPpage]    "[PyTorch] GPU 분산 학습 1 - DP / DDP / FSDP 개념".
 *
 * The problem ([Gibiansky] §Scatter-reduce, opening paragraph): N ranks each
 * hold an array of the same length P; afterwards every rank holds the same
 * array.  Here that array is the element-wise MEAN of the N inputs, because
 * data-parallel SGD averages the per-rank gradients and applies the average
 * to the weights ([Gibiansky] §The communication problem; [TrainMGPU]
 * §Training Process, steps 2-3; [DDPpage] §DDP: every rank ends with the
 * identical gradient and updates on its own).
 *
 * Numerics contract (binary32):
 *   - Chunk c of the plan's chunk table is summed in ring order, starting at
 *     rank c: ((g_c + g_{c+1}) + g_{c+2}) + ... + g_{c+N-1} (ranks mod N).
 *     That is the order the scatter-reduce of [Gibiansky] §Scatter-reduce
 *     produces (rank n starts by sending chunk n).
 *   - mean = S / N, one correctly rounded IEEE division.
 *   - SGD: w = w - (lr * mean), the product and the difference each rounded
 *     once (no fused multiply-add).
 *   - No flush of subnormals; NaN and infinity propagate.
 *   With these, every algorithm below gives bit-identical results.
 * bf16: values are widened exactly to binary32, summed and divided as above,
 * and each bf16 buffer receives the mean rounded to nearest-even; the SGD
 * update uses the binary32 mean.
 *
 * Memory and streams: every device pointer is owned by the caller and must
 * stay valid until the work enqueued on `stream` (a hipStream_t passed as
 * void*, NULL = the default stream) has finished.  Calls return after
 * enqueueing; they never synchronise, except rar_rank_stride_tune, which
 * times work on its stream and waits for it.  Rank buffers, weights and bucket
 * buffers must be 16-byte aligned; bucket tensors need only element
 * alignment.  The only device allocations are binary32 workspaces of bf16
 * rings: a bf16 plan set to RAR_ALGO_RING (rar_plan_set_algo, or a bucket call
 * that builds such a plan for itself), which lives until the plan is
 * destroyed, and a bf16 RAR_ALGO_RING bucket call over per-rank arenas (one
 * float per element of the plan, kept with the bucket handle until it is
 * destroyed).
 *
 * Graph capture: the execute and bucket calls only enqueue kernels and
 * stream waits (no allocation, synchronisation or memset), so they can be
 * captured into a HIP graph and replayed, once the plans they use exist and
 * any bf16 ring workspace has been allocated by rar_plan_set_algo.  Bucket
 * calls make their per-size plans on first use (a bf16 RAR_ALGO_RING bucket
 * call allocates the workspaces then): make one call before capturing.  The
 * ready events of a captured rar_bucket_allreduce_arena must be recorded
 * inside the same capture (on a stream forked from the capturing one).
 *
 * Errors: every argument is checked before any device work is enqueued; on
 * an argument error nothing is enqueued and a negative rar_status is
 * returned.  RAR_EHIP means a HIP launch or runtime call failed, RAR_ENOMEM
 * that a device allocation did; a call of several launches that fails that
 * way part-way may leave its earlier launches enqueued, and the buffers'
 * contents are then unspecified.  The library clears HIP's last-error state
 * when it returns either, so the caller's next HIP call does not report it
 * again.
 * Thread safety: a plan is immutable after rar_plan_set_algo; a plan without
 * a workspace may be used from several host threads and streams at once.  A
 * bf16 ring plan owns one workspace and must be used by one stream at a time.
 * A bucket handle may be used from several threads and streams at once (its
 * plan cache is locked), except with dtype bf16 and RAR_ALGO_RING, whose
 * binary32 workspaces (one per bucket size for bucket buffers, one per handle
 * for arenas) are shared by every call: one stream at a time.
 */
#ifndef RAR_H
#define RAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RAR_MAX_RANKS 64
#define RAR_MAX_STRIDE_CANDIDATES 64
/* binary32 elements of the library's static device workspace (64 MiB on each
 * device it runs on), used by rar_allreduce_ring_noalloc */
#define RAR_STATIC_WS_ELEMS (1 << 24)

typedef struct rar_plan_s *rar_plan_t;
typedef struct rar_buckets_s *rar_buckets_t;

typedef enum { RAR_F32 = 0, RAR_BF16 = 1 } rar_dtype;

/* How P elements are cut into N chunks ([Gibiansky] §Scatter-reduce: the
 * array is split into N chunks; the page does not say how when N does not
 * divide P). */
typedef enum {
    RAR_CHUNK_BALANCED = 0, /* sizes differ by at most 1, larger chunks first */
    RAR_CHUNK_CEIL = 1,     /* ceil(P/N) each; the tail takes the rest (may be short or empty) */
    RAR_CHUNK_ALIGN16 = 2   /* ceil(P/N) rounded up to whole 16-byte groups; tail as CEIL */
} rar_chunking;

typedef enum {
    RAR_ALGO_FUSED = 0, /* one pass: reads every rank once, writes every rank once */
    RAR_ALGO_RING = 1,  /* the 2(N-1) ring steps of [Gibiansky], one kernel per step */
    RAR_ALGO_NAIVE = 2  /* prior art: rank 0 reduces all and sends back ([Gibiansky]
                           §The communication problem); its own summation order */
} rar_algo;

typedef enum {
    RAR_OK = 0,
    RAR_EINVAL = -1,    /* bad argument */
    RAR_EMISMATCH = -2, /* P differs from the plan's P */
    RAR_EALIGN = -3,    /* a device pointer is not 16-byte aligned */
    RAR_ENOMEM = -4,    /* host or device allocation failed */
    RAR_EHIP = -5,      /* a HIP runtime call or kernel launch failed */
    RAR_ETOOLARGE = -6  /* P exceeds the static workspace (rar_allreduce_ring_noalloc) */
} rar_status;

/* ---------------------------------------------------------------------- */
/* Plans                                                                   */
/* ---------------------------------------------------------------------- */

/* Create a plan for N ranks (1..RAR_MAX_RANKS) of P >= 0 elements of dtype,
 * cut into chunks by `chunking` ([Gibiansky] §Scatter-reduce).  Host memory
 * only; no HIP call.  *out receives the plan (NULL on error).  The algorithm
 * starts as RAR_ALGO_FUSED. */
rar_status rar_plan(int N, int64_t P, rar_dtype dtype, rar_chunking chunking, rar_plan_t *out);

/* Not an operation of the pages: layout advice for callers that place the N
 * logical ranks of one device in a single allocation (rank n at base +
 * n * stride, base 16-byte aligned):
 * *stride_bytes receives the smallest stride >= P * element size that is
 * 2 MiB modulo 4 MiB.  Where rank buffers start matters on MI355X; measured
 * for the fused pass, 10 ranks x 300M fp32 with SGD, one process per box:
 * this stride 4.17-4.39 ms; separately allocated buffers (which lie a
 * multiple of 4 MiB apart) 4.28-4.59 ms; a stride of 1 or 3 MiB modulo
 * 4 MiB 4.40-4.80 ms.  40 ranks x 100M bf16: 2.92 ms against 3.12 ms for
 * separate buffers.  The rule does not hold for every shape: at 8 ranks x
 * 735M fp32 these strides are the slowest (8.1-8.4 ms against 7.5 ms for
 * multiples of 8 MiB), because which strides are fast follows a hash of
 * higher address bits; rar_rank_stride_tune measures instead.  Results never
 * depend on the layout.  Host only, no HIP call.  RAR_EINVAL: NULL
 * stride_bytes, unknown dtype, P < 0, or P so large that the stride
 * overflows. */
rar_status rar_rank_stride(int64_t P, rar_dtype dtype, int64_t *stride_bytes);

/* The stride candidates rar_rank_stride_tune times, so that a caller can size
 * its pool: *stride_bytes receives candidate k (0 <= k <
 * RAR_MAX_STRIDE_CANDIDATES) for ranks of P elements of dtype.  With s0 the
 * smallest multiple of 2 MiB >= P * element size, candidates 0..31 are s0,
 * s0 + 2 MiB, ..., s0 + 62 MiB, and candidates 32..63 are the multiples of
 * 8 MiB from the first one >= s0 + 64 MiB, 8 MiB apart.  They increase with
 * k; rar_rank_stride's stride is candidate 0 or 1.  A pool for the first K
 * candidates needs (N-1) * candidate(K-1) + P * element size bytes.  Host
 * only, no HIP call.  RAR_EINVAL: NULL stride_bytes, unknown dtype, P < 0, k
 * out of range, or P too large. */
rar_status rar_rank_stride_candidate(int64_t P, rar_dtype dtype, int k, int64_t *stride_bytes);

/* Not an operation of the pages either: measured layout advice for the same
 * single-allocation placement.  Times the fused mean over N ranks carved
 * from `pool` (device, 16-byte aligned, pool_bytes long) at the strides
 * rar_rank_stride_candidate gives, the first max_candidates
 * (1..RAR_MAX_STRIDE_CANDIDATES) of them for which (N-1) * stride + P *
 * element size <= pool_bytes, and returns the fastest in *stride_bytes.
 * Two stages, each in rounds that visit the candidates
 * forward and backward in turn, one untimed and two timed calls per
 * candidate and round: four rounds over every candidate, then eight more
 * over the finalists, the four with the smallest medians so far and the
 * stride rar_rank_stride gives when it is a candidate (24 timings each).
 * The finalist with the smallest median wins, ties to the smaller stride --
 * except that rar_rank_stride's stride is kept if its median exceeds the
 * winner's by no more than a third of the finalists' typical spread (the
 * median of their spreads, each the range of the middle three quarters of
 * its timings), about two standard errors of a difference of two such
 * medians: on MI355X the fast strides lie within about 1% of each other,
 * about as much as single calls vary.  Fast strides also lie beyond the
 * first few: at 10 x 300M fp32 the best of a sweep from 1146 to 1658 MiB
 * were 1280 and 1368 MiB, the SGD call 1% faster there than at the best
 * stride within 1146-1272 MiB and 2.5% faster than at the static rule's
 * 1146 MiB (one box, interleaved rounds).  The
 * pool's contents are overwritten; the call enqueues on `stream` and waits
 * for it, so it must not run under graph capture.  N == 1 or P == 0 returns
 * s0 without device work.  Which strides are fast differs by shape (see
 * rar_rank_stride); measured on MI355X, 8 ranks x 735M fp32: 7.50-7.57 ms at
 * the pick against 7.86 ms for separate allocations and 8.35 ms for
 * rar_rank_stride.  RAR_EINVAL: NULL stride_bytes or pool, N outside
 * 1..RAR_MAX_RANKS, P < 0, unknown dtype, max_candidates out of range, or a
 * pool too small for even s0.  RAR_EALIGN: pool not 16-byte aligned.
 * RAR_EHIP / RAR_ENOMEM: a HIP call failed. */
rar_status rar_rank_stride_tune(int N, int64_t P, rar_dtype dtype, void *pool, int64_t pool_bytes,
                                int max_candidates, void *stream, int64_t *stride_bytes);

/* rar_rank_stride_tune, also reporting what it measured: *n_candidates
 * receives K, the number of candidates timed (0 when N == 1 or P == 0), and
 * for k < K cand_stride[k], median_ms[k] and spread_ms[k], over all of
 * candidate k's timings (8, or 24 for a finalist; the spread is the range of
 * their middle three quarters).  The arrays hold max_candidates entries; any
 * of these outputs may be NULL. */
rar_status rar_rank_stride_tune_stats(int N, int64_t P, rar_dtype dtype, void *pool, int64_t pool_bytes,
                                      int max_candidates, void *stream, int64_t *stride_bytes,
                                      int *n_candidates, int64_t cand_stride[], float median_ms[],
                                      float spread_ms[]);

/* Free the plan and its workspace (if any).  Waits for the device to finish
 * work that may use the workspace.  NULL is accepted. */
rar_status rar_plan_destroy(rar_plan_t plan);

/* Select the algorithm used by rar_allreduce_mean / rar_allreduce_sgd.
 * For a bf16 plan, RAR_ALGO_RING allocates the binary32 workspace (4*P
 * bytes, chunk-indexed: it carries the running partial sum of each chunk
 * between ring steps); RAR_ENOMEM if that fails.  RAR_ALGO_NAIVE is
 * supported for RAR_F32 only. */
rar_status rar_plan_set_algo(rar_plan_t plan, rar_algo algo);

/* Kernel launch shape: at most max_blocks workgroups per launch (0 = the
 * library's choice).  Results do not depend on it. */
rar_status rar_plan_set_grid(rar_plan_t plan, int max_blocks);

/* Chunk c: element offset and length, and the rank that holds the finished
 * chunk after scatter-reduce, (c-1) mod N (derived from [Gibiansky]
 * §Scatter-reduce, and the step-1 table of §Allgather where GPU n starts by
 * sending chunk n+1).  Any output pointer may be NULL. */
rar_status rar_plan_chunk(rar_plan_t plan, int c, int64_t *offset, int64_t *length, int *owner_rank);

/* Elements rank `rank` sends and receives in the ring schedule (N-1
 * scatter-reduce plus N-1 all-gather transfers, [Gibiansky] §Allreduce
 * communication cost): 2P - |C(rank+1)| - |C(rank+2)| sent and
 * 2P - |C(rank)| - |C(rank+1)| received, i.e. 2(N-1)P/N when N divides P. */
rar_status rar_plan_traffic(rar_plan_t plan, int rank, int64_t *sent_elems, int64_t *recv_elems);

/* ---------------------------------------------------------------------- */
/* All-reduce                                                              */
/* ---------------------------------------------------------------------- */

/* In place: every bufs[n] (n < N; device, P elements of the plan's dtype)
 * ends holding the element-wise mean of the N inputs.  bufs is a host
 * array of N device pointers; it is copied, so it need not outlive the
 * call.  The N buffers must not overlap.  P must equal the plan's P (it is
 * passed again as a check: RAR_EMISMATCH).  P == 0 is a no-op. */
rar_status rar_allreduce_mean(rar_plan_t plan, void *const bufs[], int64_t P, void *stream);

/* As rar_allreduce_mean, then the synchronous SGD step on the binary32
 * weights w (device, P floats, must not overlap any buffer):
 * w[e] = w[e] - lr * mean[e] ([Gibiansky] §The communication problem;
 * [TrainMGPU] §Training Process, step 3; [DDPpage] §DDP). */
rar_status rar_allreduce_sgd(rar_plan_t plan, void *const bufs[], float *w, float lr, int64_t P,
                             void *stream);

/* Scatter-reduce with the owner's update, then an all-gather of weights (the
 * sharded shape of [DDPpage] §FSDP: gradients are reduce-scattered and each
 * rank updates only the part it owns).  After the call:
 *   - the owner of chunk c, (c-1) mod N, holds mean[C_c] in bufs[owner][C_c];
 *     other parts of the gradient buffers hold ring partial sums (unspecified);
 *   - every weight replica w_reps[n] (device, P floats each) holds
 *     w_reps[owner][e] - lr*mean[e] for every element e, i.e. the same bits
 *     rar_allreduce_sgd gives when all replicas start equal.
 * Only RAR_F32 plans; the algorithm selected by set_algo is ignored (this
 * call is always the ring: N-1 scatter-reduce steps, N-1 all-gather steps). */
rar_status rar_reduce_scatter_sgd_allgather(rar_plan_t plan, void *const bufs[],
                                            float *const w_reps[], float lr, int64_t P,
                                            void *stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The ring
 * algorithm of rar_allreduce_mean (w == NULL) or rar_allreduce_sgd (w != NULL)
 * with the same arguments, results and checks, whatever algorithm the plan
 * has selected, and with no device allocation, free or memset: a bf16 plan's
 * binary32 partial sums go to a workspace the library holds in a static device
 * array of RAR_STATIC_WS_ELEMS floats instead of one the plan allocates
 * (binary32 plans need none).  Each device keeps its own copy of that array
 * until the process ends; its address is looked up once per device, on the
 * first call there.  Every element of the workspace that a call reads was
 * written earlier in the same call, so nothing is cleared between calls.  All
 * calls on one device share the array: calls on that device that overlap in
 * time (other streams, other host threads) race and must be serialised by the
 * caller.  `stream` must belong to the current device (RAR_EINVAL otherwise).
 * RAR_ETOOLARGE: a bf16 plan with N > 1 and P > RAR_STATIC_WS_ELEMS. */
rar_status rar_allreduce_ring_noalloc(rar_plan_t plan, void *const bufs[], float *w, float lr, int64_t P,
                                      void *stream);

/* ---------------------------------------------------------------------- */
/* Buckets: a ragged list of per-layer gradients reduced in fixed-size     */
/* buckets ([Gibiansky] §Applying allreduce to deep learning: the          */
/* all-reduce can run on a subset of the parameters, and output-layer      */
/* gradients are ready first).                                             */
/* ---------------------------------------------------------------------- */

/* Lay n_tensors tensors (numel[t] elements each, listed in the order
 * back-propagation produces them) end to end and cut the stream into
 * buckets of bucket_bytes / sizeof(dtype) elements; a tensor that crosses a
 * boundary is split.  Host memory only. */
rar_status rar_bucket_plan(int n_tensors, const int64_t numel[], rar_dtype dtype, int64_t bucket_bytes,
                           rar_buckets_t *out);

rar_status rar_bucket_destroy(rar_buckets_t b);

/* Number of buckets and the largest bucket's element count. */
rar_status rar_bucket_count(rar_buckets_t b, int *n_buckets, int64_t *max_bucket_elems);

/* Bucket `bucket`: its first element in the concatenated stream, its element
 * count and its number of segments.  Any output may be NULL. */
rar_status rar_bucket_info(rar_buckets_t b, int bucket, int64_t *stream_offset, int64_t *elems,
                           int *n_segments);

/* Segment `seg` of a bucket: tensor index, offset inside that tensor, offset
 * inside the bucket, length (elements).  Any output may be NULL. */
rar_status rar_bucket_segment(rar_buckets_t b, int bucket, int seg, int *tensor, int64_t *tensor_offset,
                              int64_t *bucket_offset, int64_t *length);

/* Copy the bucket's segments of every rank's tensors into bucket_bufs[n]
 * (device, >= the bucket's elements).  tensors is a host array of N*n_tensors
 * device pointers, rank-major: tensors[n*n_tensors + t].  The N ranks' copies
 * of a segment, and the bucket's elements of the N bucket buffers, must all be
 * disjoint memory (RAR_EINVAL otherwise). */
rar_status rar_bucket_pack(rar_buckets_t b, int bucket, int N, void *const tensors[],
                           void *const bucket_bufs[], void *stream);

/* The reverse copy, from bucket_bufs[n] back into the tensors (same checks). */
rar_status rar_bucket_unpack(rar_buckets_t b, int bucket, int N, void *const bucket_bufs[],
                             void *const tensors[], void *stream);

/* Every bucket in order, all-reduce-mean in place in the tensors.  Element e
 * of a bucket ends bit-identical to what rar_allreduce_mean gives for that
 * bucket alone (chunk table of the bucket's size, `chunking`).
 * With RAR_ALGO_FUSED and N in {2, 4, 8, 10, 16, 40} the reduction reads and
 * writes the tensors directly (each bucket segment cut at the bucket's chunk
 * boundaries, and the pieces of consecutive tensors in one chunk joined
 * where every rank's tensors are adjacent in memory; 2*N*size bytes moved
 * per bucket) and bucket_bufs may be NULL.
 * The jobs of consecutive buckets then share launches, so all N*n_tensors
 * tensors must be pairwise disjoint memory (RAR_EINVAL otherwise).
 * With RAR_ALGO_RING, RAR_F32 and N >= 2 the 2(N-1) ring steps of
 * [Gibiansky] §Scatter-reduce and §Allgather run on those same pieces in
 * place (5*(N-1)*size*4 bytes moved per bucket, no packing); each step is
 * a few launches over the pieces of every bucket, so the tensors must again
 * be pairwise disjoint, and bucket_bufs may be NULL.  When every rank's
 * tensors lie end to end in the plan's order (views of one flat buffer per
 * rank, 16-byte aligned, with 16-byte aligned bucket starts), the call runs
 * as rar_bucket_allreduce_arena over those buffers, also for bf16 with
 * RAR_ALGO_RING (no packing; binary32 partial sums in a workspace kept with
 * the bucket handle).
 * Otherwise each bucket is packed into bucket_bufs[n] (N device buffers of at
 * least max_bucket_elems elements, 16-byte aligned, reused by every bucket,
 * overlapping neither each other nor the tensors: RAR_EINVAL), reduced with
 * `algo`, and unpacked. */
rar_status rar_bucket_allreduce_mean(rar_buckets_t b, int N, rar_chunking chunking, rar_algo algo,
                                     void *const tensors[], void *const bucket_bufs[], void *stream);

/* Every bucket in order, in place over per-rank flat arenas, each bucket
 * starting only once its gradients exist ([Gibiansky] §Applying allreduce to
 * deep learning: back-propagation produces the output layers' gradients
 * first, so their reduction can overlap the rest of the backward pass).
 * arenas[n] (device, 16-byte aligned) holds rank n's tensors end to end in
 * the plan's order, so bucket k is the slice [stream_offset, +elems) of every
 * arena and needs no packing.  ready_events is a host array of n_buckets
 * hipEvent_t (as void*), or NULL: before bucket k the call makes `stream`
 * wait for ready_events[k] (a NULL entry waits for nothing).  The producer
 * records the events on its own stream; the waits are enqueued, the call
 * does not block the host.  Every bucket start must be 16-byte aligned
 * (RAR_EALIGN otherwise; a bucket size that is a multiple of 16 bytes gives
 * that), and the N arenas (total elements each) must not overlap
 * (RAR_EINVAL).  With RAR_ALGO_FUSED and N in {2, 4, 8, 10, 16, 40}, and
 * with RAR_ALGO_RING and N >= 2 (each ring step over every chunk of those
 * buckets at once; bf16 keeps the binary32 partial sums in a workspace of one
 * float per element, allocated on the first such call and kept with the
 * bucket handle), the buckets between two ready events share launches.
 * Results are bit-identical to rar_allreduce_mean on each slice. */
rar_status rar_bucket_allreduce_arena(rar_buckets_t b, int N, rar_chunking chunking, rar_algo algo,
                                      void *const arenas[], void *const ready_events[], void *stream);

/* ---------------------------------------------------------------------- */

/* Static description of a status code; never NULL. */
const char *rar_strerror(rar_status s);

/* Library version as major*10000 + minor*100 + patch (0.2.0 = 200 adds
 * rar_rank_stride, 0.3.0 = 300 rar_rank_stride_tune, 0.4.0 = 400
 * rar_allreduce_ring_noalloc, 0.5.0 = 500 rar_rank_stride_tune_stats,
 * 0.6.0 = 600 rar_rank_stride_candidate and the wider stride search). */
int rar_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RAR_H */
