// rar_host.cpp -- host side of librar.so: plans, argument checks, the launch
// sequences of each algorithm, and the bucketer.  No device work is enqueued
// before every argument has been checked.
//
// Sources: [Gibiansky] "Bringing HPC Techniques to Deep Learning" (A.
// Gibiansky, Baidu SVAIL), sections "Scatter-reduce", "Allgather",
// "Allreduce communication cost", "Applying allreduce to deep learning",
// "The communication problem"; [DDPpage] "[PyTorch] GPU 분산 학습 1 - DP / DDP
// / FSDP 개념", sections "DDP" and "FSDP".
#include <algorithm>
#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "rar_internal.h"

using rar::kMaxRanks;
constexpr int kMaxStrideCandidates = RAR_MAX_STRIDE_CANDIDATES;

struct rar_plan_s {
    int N = 0;
    int64_t P = 0;
    rar_dtype dtype = RAR_F32;
    rar_chunking chunking = RAR_CHUNK_BALANCED;
    rar_algo algo = RAR_ALGO_FUSED;
    int max_blocks = 0;          // 0: default
    rar::ChunkTable ct{};
    int64_t max_chunk = 0;
    float *ws = nullptr;         // bf16 ring: binary32 chunk-indexed partial sums
};

namespace {

constexpr int kDefaultBlocks = 1 << 24;  // no cap: one tile per workgroup (x is capped at 2^22 - 1 per job)

int elem_bytes(rar_dtype d) { return d == RAR_BF16 ? 2 : 4; }

bool valid_dtype(int d) { return d == RAR_F32 || d == RAR_BF16; }

// Chunk table per rar_chunking (see rar.h).
void cut_chunks(int N, int64_t P, rar_chunking mode, int es, rar::ChunkTable &ct)
{
    if (mode == RAR_CHUNK_BALANCED) {
        const int64_t q = P / N, r = P % N;
        for (int c = 0; c <= N; ++c)
            ct.off[c] = c * q + std::min<int64_t>(c, r);
        return;
    }
    int64_t len = (P + N - 1) / N;
    if (mode == RAR_CHUNK_ALIGN16) {
        const int64_t g = 16 / es;
        len = (len + g - 1) / g * g;
    }
    for (int c = 0; c < N; ++c)
        ct.off[c] = std::min<int64_t>(c * len, P);
    ct.off[N] = P;
}

int block_budget(const rar_plan_s *pl) { return pl->max_blocks > 0 ? pl->max_blocks : kDefaultBlocks; }

// Stride candidates of the layout tuner for ranks of `need` bytes: the first
// kFineCandidates at 2 MiB steps from s0 (the smallest multiple of 2 MiB >=
// need), then multiples of 8 MiB from the first one >= s0 + 2 MiB *
// kFineCandidates, at 8 MiB steps.  Measured on MI355X the fast strides lie
// both near s0 and further out, and those further out are multiples of 8 MiB.
constexpr int kFineCandidates = 32;
constexpr int64_t kMiB = int64_t(1) << 20;

int64_t stride_base(int64_t need) { return std::max<int64_t>(2 * kMiB, (need + 2 * kMiB - 1) / (2 * kMiB) * (2 * kMiB)); }

int64_t stride_candidate(int64_t s0, int k)
{
    if (k < kFineCandidates)
        return s0 + 2 * kMiB * k;
    const int64_t c0 = (s0 + 2 * kMiB * kFineCandidates + 8 * kMiB - 1) / (8 * kMiB) * (8 * kMiB);
    return c0 + 8 * kMiB * (k - kFineCandidates);
}

rar_status hip_status(hipError_t e) { return e == hipSuccess ? RAR_OK : RAR_EHIP; }

// A failed HIP runtime call also sets HIP's per-thread "last error", which
// the caller's next HIP call (a torch kernel launch, say) would report as its
// own.  The library maps the failure to a status and clears it.
rar_status hip_failed(hipError_t e)
{
    (void)hipGetLastError();
    return e == hipErrorOutOfMemory ? RAR_ENOMEM : RAR_EHIP;
}

// No C++ exception crosses the C ABI: the entry points that build host
// containers run their body through this (allocation failure -> RAR_ENOMEM).
template <class F>
rar_status no_throw(F &&body)
{
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return RAR_ENOMEM;
    } catch (...) {
        return RAR_EINVAL;
    }
}

struct Range {
    uintptr_t lo, hi;
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks shared by every execute call.  P == 0 returns RAR_OK early through
// *noop without looking at the pointers (empty tensors may have none).
rar_status check_exec(const rar_plan_s *pl, void *const bufs[], int64_t P, bool *noop)
{
    *noop = false;
    if (!pl || !bufs)
        return RAR_EINVAL;
    if (P != pl->P)
        return RAR_EMISMATCH;
    if (P == 0) {
        *noop = true;
        return RAR_OK;
    }
    const uintptr_t bytes = (uintptr_t)P * elem_bytes(pl->dtype);
    for (int n = 0; n < pl->N; ++n) {
        if (!bufs[n])
            return RAR_EINVAL;
        if ((uintptr_t)bufs[n] & 15)
            return RAR_EALIGN;
    }
    for (int i = 0; i < pl->N; ++i)
        for (int j = i + 1; j < pl->N; ++j)
            if (overlaps({(uintptr_t)bufs[i], (uintptr_t)bufs[i] + bytes},
                         {(uintptr_t)bufs[j], (uintptr_t)bufs[j] + bytes}))
                return RAR_EINVAL;
    return RAR_OK;
}

rar_status check_weights(const rar_plan_s *pl, void *const bufs[], const float *w)
{
    if (!w)
        return RAR_EINVAL;
    if ((uintptr_t)w & 15)
        return RAR_EALIGN;
    const uintptr_t bytes = (uintptr_t)pl->P * elem_bytes(pl->dtype);
    const Range wr{(uintptr_t)w, (uintptr_t)w + (uintptr_t)pl->P * 4};
    for (int n = 0; n < pl->N; ++n)
        if (overlaps(wr, {(uintptr_t)bufs[n], (uintptr_t)bufs[n] + bytes}))
            return RAR_EINVAL;
    return RAR_OK;
}

// --- launch sequences --------------------------------------------------------

rar_status run_fused(const rar_plan_s *pl, void *const bufs[], float *w, float lr, hipStream_t st)
{
    rar::FusedParams p{};
    for (int n = 0; n < pl->N; ++n)
        p.bufs.p[n] = bufs[n];
    p.ct = pl->ct;
    p.w = w;
    p.lr = lr;
    p.N = pl->N;
    return hip_status(rar::launch_fused(pl->dtype, p, block_budget(pl), pl->max_chunk, st));
}

// All-gather steps ([Gibiansky] §Allgather): at step s chunk c moves from rank
// (c+s-1) mod N to rank (c+s) mod N, overwriting.  ptrs are the arrays moved
// (gradient buffers, or weight replicas), es their element size.
rar_status run_allgather(const rar_plan_s *pl, void *const ptrs[], int es, hipStream_t st)
{
    const int N = pl->N;
    for (int s = 0; s < N - 1; ++s) {
        rar::CopyParams cp{};
        cp.unit = es;
        for (int c = 0; c < N; ++c) {
            const int src = (c + s - 1 + N) % N, dst = (c + s) % N;
            const int64_t off = pl->ct.off[c], len = pl->ct.off[c + 1] - off;
            cp.job[cp.njobs++] = {static_cast<const char *>(ptrs[src]) + off * es,
                                  static_cast<char *>(ptrs[dst]) + off * es, len * es};
        }
        hipError_t e = rar::launch_copy(cp, block_budget(pl), pl->max_chunk * es, st);
        if (e != hipSuccess)
            return RAR_EHIP;
    }
    return RAR_OK;
}

// Scatter-reduce steps ([Gibiansky] §Scatter-reduce); the last one divides by
// N at the owner and, with SGD, updates the owner's chunk of the weights.
rar_status run_scatter_reduce(const rar_plan_s *pl, void *const bufs[], float *w, float *const wreps[],
                              float lr, bool sgd, hipStream_t st)
{
    const int N = pl->N;
    rar::StepParams p{};
    for (int n = 0; n < N; ++n) {
        p.bufs.p[n] = bufs[n];
        if (wreps)
            p.wreps.p[n] = wreps[n];
    }
    p.ct = pl->ct;
    p.w = w;
    p.ws = pl->ws;
    p.lr = lr;
    p.N = N;
    p.sharded = wreps ? 1 : 0;
    for (int s = 0; s < N - 1; ++s) {
        p.s = s;
        hipError_t e = rar::launch_sr_step(pl->dtype, p, s == 0, s == N - 2, sgd, block_budget(pl),
                                           pl->max_chunk, st);
        if (e != hipSuccess)
            return RAR_EHIP;
    }
    return RAR_OK;
}

rar_status run_ring(const rar_plan_s *pl, void *const bufs[], float *w, float lr, hipStream_t st)
{
    if (pl->N == 1)  // no transfers: the mean of one rank is its gradient
        return run_fused(pl, bufs, w, lr, st);
    rar_status rc = run_scatter_reduce(pl, bufs, w, nullptr, lr, w != nullptr, st);
    if (rc != RAR_OK)
        return rc;
    return run_allgather(pl, bufs, elem_bytes(pl->dtype), st);
}

// Single reducer ([Gibiansky] §The communication problem): rank 0 receives
// every other rank's gradient in turn, averages, updates, and sends the mean
// back to every rank.
rar_status run_naive(const rar_plan_s *pl, void *const bufs[], float *w, float lr, hipStream_t st)
{
    const int N = pl->N;
    if (N == 1)
        return run_fused(pl, bufs, w, lr, st);
    rar::PairParams p{};
    for (int n = 0; n < N; ++n)
        p.bufs.p[n] = bufs[n];
    p.w = w;
    p.lr = lr;
    p.N = N;
    p.P = pl->P;
    for (int src = 1; src < N; ++src) {
        p.src = src;
        hipError_t e = rar::launch_pair_add(p, src == N - 1, w != nullptr, block_budget(pl), st);
        if (e != hipSuccess)
            return RAR_EHIP;
    }
    rar::CopyParams cp{};
    cp.unit = 4;
    for (int n = 1; n < N; ++n)
        cp.job[cp.njobs++] = {bufs[0], bufs[n], pl->P * 4};
    return hip_status(rar::launch_copy(cp, block_budget(pl), pl->P * 4, st));
}

rar_status execute(rar_plan_s *pl, void *const bufs[], float *w, float lr, hipStream_t st)
{
    switch (pl->algo) {
    case RAR_ALGO_FUSED: return run_fused(pl, bufs, w, lr, st);
    case RAR_ALGO_RING: return run_ring(pl, bufs, w, lr, st);
    case RAR_ALGO_NAIVE: return run_naive(pl, bufs, w, lr, st);
    }
    return RAR_EINVAL;
}

}  // namespace

// =============================================================================
// Plans
// =============================================================================

extern "C" rar_status rar_plan(int N, int64_t P, rar_dtype dtype, rar_chunking chunking, rar_plan_t *out)
{
    if (!out)
        return RAR_EINVAL;
    *out = nullptr;
    if (N < 1 || N > kMaxRanks || P < 0 || !valid_dtype(dtype))
        return RAR_EINVAL;
    if (chunking != RAR_CHUNK_BALANCED && chunking != RAR_CHUNK_CEIL && chunking != RAR_CHUNK_ALIGN16)
        return RAR_EINVAL;
    rar_plan_s *pl = new (std::nothrow) rar_plan_s;
    if (!pl)
        return RAR_ENOMEM;
    pl->N = N;
    pl->P = P;
    pl->dtype = dtype;
    pl->chunking = chunking;
    cut_chunks(N, P, chunking, elem_bytes(dtype), pl->ct);
    for (int c = 0; c < N; ++c)
        pl->max_chunk = std::max(pl->max_chunk, pl->ct.off[c + 1] - pl->ct.off[c]);
    *out = pl;
    return RAR_OK;
}

extern "C" rar_status rar_rank_stride(int64_t P, rar_dtype dtype, int64_t *stride_bytes)
{
    constexpr int64_t MiB = int64_t(1) << 20;
    if (!stride_bytes || !valid_dtype(dtype) || P < 0 || P > (INT64_MAX - 8 * MiB) / elem_bytes(dtype))
        return RAR_EINVAL;
    const int64_t need = P * elem_bytes(dtype);
    const int64_t extra = need > 2 * MiB ? need - 2 * MiB : 0;
    *stride_bytes = 2 * MiB + (extra + 4 * MiB - 1) / (4 * MiB) * (4 * MiB);
    return RAR_OK;
}

extern "C" rar_status rar_rank_stride_candidate(int64_t P, rar_dtype dtype, int k, int64_t *stride_bytes)
{
    if (!stride_bytes || !valid_dtype(dtype) || P < 0 || k < 0 || k >= kMaxStrideCandidates ||
        P > (INT64_MAX / 4) / elem_bytes(dtype))
        return RAR_EINVAL;
    *stride_bytes = stride_candidate(stride_base(P * elem_bytes(dtype)), k);
    return RAR_OK;
}

extern "C" rar_status rar_rank_stride_tune(int N, int64_t P, rar_dtype dtype, void *pool, int64_t pool_bytes,
                                           int max_candidates, void *stream, int64_t *stride_bytes)
{
    return rar_rank_stride_tune_stats(N, P, dtype, pool, pool_bytes, max_candidates, stream, stride_bytes, nullptr,
                                      nullptr, nullptr, nullptr);
}

extern "C" rar_status rar_rank_stride_tune_stats(int N, int64_t P, rar_dtype dtype, void *pool, int64_t pool_bytes,
                                                 int max_candidates, void *stream, int64_t *stride_bytes,
                                                 int *n_candidates, int64_t cand_stride[], float median_ms[],
                                                 float spread_ms[])
{
    if (!stride_bytes || N < 1 || N > kMaxRanks || P < 0 || !valid_dtype(dtype) || max_candidates < 1 ||
        max_candidates > kMaxStrideCandidates || pool_bytes < 0 || P > (INT64_MAX / 4) / elem_bytes(dtype))
        return RAR_EINVAL;
    const int64_t need = P * elem_bytes(dtype);
    const int64_t s0 = stride_base(need);
    if (n_candidates)
        *n_candidates = 0;
    if (N == 1 || P == 0) {  // nothing to place relative to anything
        *stride_bytes = s0;
        return RAR_OK;
    }
    if (!pool)
        return RAR_EINVAL;
    if ((uintptr_t)pool & 15)
        return RAR_EALIGN;
    int K = 0;  // candidates whose N ranks fit in the pool
    while (K < max_candidates && need <= pool_bytes && stride_candidate(s0, K) <= (pool_bytes - need) / (N - 1))
        ++K;
    if (K == 0)
        return RAR_EINVAL;

    rar_plan_t pl = nullptr;
    rar_status rc = rar_plan(N, P, dtype, RAR_CHUNK_BALANCED, &pl);
    if (rc != RAR_OK)
        return rc;
    hipEvent_t ev[2] = {nullptr, nullptr};
    for (hipEvent_t &e : ev) {
        const hipError_t he = hipEventCreate(&e);
        if (he != hipSuccess && rc == RAR_OK)
            rc = hip_failed(he);
    }
    // Two stages.  Stage 1 times every candidate in four rounds, alternately
    // forward and backward over the candidates (so a drift in the device's
    // speed reaches all of them alike); per candidate and round one untimed
    // call, then two timed ones.  The fast strides lie within ~1% of each
    // other and single calls vary by about as much, so stage 2 times the
    // finalists -- the four with the smallest stage-1 medians, and the static
    // rule's stride -- in eight more rounds the same way: 24 timings each.
    constexpr int kRounds1 = 4, kRounds2 = 8, kTimed = 2, kFinalists = 4;
    constexpr int kMaxSamples = (kRounds1 + kRounds2) * kTimed;
    float ms[kMaxStrideCandidates][kMaxSamples] = {};
    int ns[kMaxStrideCandidates] = {};
    void *bufs[kMaxRanks];
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto time_candidate = [&](int k) {
        for (int n = 0; n < N; ++n)
            bufs[n] = static_cast<char *>(pool) + (int64_t)n * stride_candidate(s0, k);
        rc = rar_allreduce_mean(pl, bufs, P, stream);
        for (int t = 0; t < kTimed && rc == RAR_OK; ++t) {
            hipError_t he = hipEventRecord(ev[0], st);
            if (he == hipSuccess && (rc = rar_allreduce_mean(pl, bufs, P, stream)) != RAR_OK)
                break;
            if (he == hipSuccess)
                he = hipEventRecord(ev[1], st);
            if (he == hipSuccess)
                he = hipEventSynchronize(ev[1]);
            if (he == hipSuccess)
                he = hipEventElapsedTime(&ms[k][ns[k]++], ev[0], ev[1]);
            if (he != hipSuccess)
                rc = hip_failed(he);
        }
    };
    // per candidate: the median of its timings (the mean of the middle two)
    // and their spread (the range of the middle three quarters)
    float med[kMaxStrideCandidates] = {}, spread[kMaxStrideCandidates] = {};
    auto summarise = [&](int k) {
        float t[kMaxSamples];
        const int n = ns[k];
        std::copy(ms[k], ms[k] + n, t);
        std::sort(t, t + n);
        med[k] = 0.5f * (t[n / 2 - 1] + t[n / 2]);
        spread[k] = t[n - 1 - n / 8] - t[n / 8];
    };
    for (int r = 0; r < kRounds1 && rc == RAR_OK; ++r)
        for (int i = 0; i < K && rc == RAR_OK; ++i)
            time_candidate(r % 2 == 0 ? i : K - 1 - i);
    int64_t fixed = 0;
    (void)rar_rank_stride(P, dtype, &fixed);
    int si = -1;
    for (int k = 0; k < K; ++k)
        if (stride_candidate(s0, k) == fixed)
            si = k;
    const bool static_is_candidate = si >= 0;
    int fin[kFinalists + 1], nfin = 0;
    if (rc == RAR_OK) {
        int order[kMaxStrideCandidates];
        for (int k = 0; k < K; ++k) {
            summarise(k);
            order[k] = k;
        }
        std::stable_sort(order, order + K, [&](int a, int b) { return med[a] < med[b]; });
        for (int i = 0; i < std::min(K, kFinalists); ++i)
            fin[nfin++] = order[i];
        if (static_is_candidate && std::find(fin, fin + nfin, si) == fin + nfin)
            fin[nfin++] = si;
        std::sort(fin, fin + nfin);
    }
    for (int r = 0; r < kRounds2 && rc == RAR_OK; ++r)
        for (int i = 0; i < nfin && rc == RAR_OK; ++i)
            time_candidate(fin[r % 2 == 0 ? i : nfin - 1 - i]);
    if (rc == RAR_OK) {
        // The finalist with the smallest median over its 24 timings wins
        // (ties to the smaller stride) -- unless the static rule's stride
        // exceeds it by no more than a third of the finalists' typical spread
        // (the median of their spreads).  That is about two standard errors
        // of a difference of two medians of 24 timings (the middle three
        // quarters span about 2.3 standard deviations of one timing, and the
        // median of 24 has a standard error of about a quarter of one), so a
        // smaller gap is not a measured improvement and the static stride
        // stays.  The typical spread, not the static stride's own, is the
        // yardstick: a layout whose calls vary more than the others' is
        // itself the slower one, and the static stride at 10 x 300M is one.
        float fs[kFinalists + 1];
        int best = fin[0];
        for (int i = 0; i < nfin; ++i) {
            summarise(fin[i]);
            fs[i] = spread[fin[i]];
            if (med[fin[i]] < med[best])
                best = fin[i];
        }
        std::sort(fs, fs + nfin);
        const float typical = nfin % 2 ? fs[nfin / 2] : 0.5f * (fs[nfin / 2 - 1] + fs[nfin / 2]);
        if (static_is_candidate && si != best && med[si] - med[best] <= typical / 3.0f)
            best = si;
        *stride_bytes = stride_candidate(s0, best);
        if (n_candidates)
            *n_candidates = K;
        for (int k = 0; k < K; ++k) {
            if (cand_stride)
                cand_stride[k] = stride_candidate(s0, k);
            if (median_ms)
                median_ms[k] = med[k];
            if (spread_ms)
                spread_ms[k] = spread[k];
        }
    }
    for (hipEvent_t e : ev)
        if (e)
            (void)hipEventDestroy(e);
    rar_plan_destroy(pl);
    return rc;
}

extern "C" rar_status rar_plan_destroy(rar_plan_t plan)
{
    if (!plan)
        return RAR_OK;
    rar_status rc = RAR_OK;
    if (plan->ws) {
        const hipError_t e = hipFree(plan->ws);
        if (e != hipSuccess)
            rc = hip_failed(e);
    }
    delete plan;
    return rc;
}

extern "C" rar_status rar_plan_set_algo(rar_plan_t plan, rar_algo algo)
{
    if (!plan)
        return RAR_EINVAL;
    if (algo != RAR_ALGO_FUSED && algo != RAR_ALGO_RING && algo != RAR_ALGO_NAIVE)
        return RAR_EINVAL;
    if (algo == RAR_ALGO_NAIVE && plan->dtype != RAR_F32)
        return RAR_EINVAL;
    if (algo == RAR_ALGO_RING && plan->dtype == RAR_BF16 && !plan->ws && plan->P > 0 && plan->N > 1) {
        void *p = nullptr;
        const hipError_t e = hipMalloc(&p, (size_t)plan->P * sizeof(float));
        if (e != hipSuccess)
            return hip_failed(e);
        plan->ws = static_cast<float *>(p);
    }
    plan->algo = algo;
    return RAR_OK;
}

extern "C" rar_status rar_plan_set_grid(rar_plan_t plan, int max_blocks)
{
    if (!plan || max_blocks < 0)
        return RAR_EINVAL;
    plan->max_blocks = max_blocks;
    return RAR_OK;
}

extern "C" rar_status rar_plan_chunk(rar_plan_t plan, int c, int64_t *offset, int64_t *length, int *owner_rank)
{
    if (!plan || c < 0 || c >= plan->N)
        return RAR_EINVAL;
    if (offset)
        *offset = plan->ct.off[c];
    if (length)
        *length = plan->ct.off[c + 1] - plan->ct.off[c];
    if (owner_rank)
        *owner_rank = (c - 1 + plan->N) % plan->N;
    return RAR_OK;
}

extern "C" rar_status rar_plan_traffic(rar_plan_t plan, int rank, int64_t *sent_elems, int64_t *recv_elems)
{
    if (!plan || rank < 0 || rank >= plan->N)
        return RAR_EINVAL;
    const int N = plan->N;
    int64_t sent = 0, recv = 0;
    // walk the schedule: scatter-reduce sends chunk (n-s), all-gather (n+1-s);
    // the rank receives what its left neighbour sends
    for (int phase = 0; phase < 2; ++phase) {
        for (int s = 0; s < N - 1; ++s) {
            const int cs = ((rank + phase - s) % N + N) % N;
            const int cr = ((rank - 1 + phase - s) % N + N) % N;
            sent += plan->ct.off[cs + 1] - plan->ct.off[cs];
            recv += plan->ct.off[cr + 1] - plan->ct.off[cr];
        }
    }
    if (sent_elems)
        *sent_elems = sent;
    if (recv_elems)
        *recv_elems = recv;
    return RAR_OK;
}

// =============================================================================
// All-reduce
// =============================================================================

extern "C" rar_status rar_allreduce_mean(rar_plan_t plan, void *const bufs[], int64_t P, void *stream)
{
    bool noop;
    rar_status rc = check_exec(plan, bufs, P, &noop);
    if (rc != RAR_OK || noop)
        return rc;
    return execute(plan, bufs, nullptr, 0.0f, static_cast<hipStream_t>(stream));
}

extern "C" rar_status rar_allreduce_sgd(rar_plan_t plan, void *const bufs[], float *w, float lr, int64_t P,
                                        void *stream)
{
    bool noop;
    rar_status rc = check_exec(plan, bufs, P, &noop);
    if (rc != RAR_OK || noop)
        return rc;
    rc = check_weights(plan, bufs, w);
    if (rc != RAR_OK)
        return rc;
    return execute(plan, bufs, w, lr, static_cast<hipStream_t>(stream));
}

extern "C" rar_status rar_reduce_scatter_sgd_allgather(rar_plan_t plan, void *const bufs[],
                                                       float *const w_reps[], float lr, int64_t P,
                                                       void *stream)
{
    bool noop;
    rar_status rc = check_exec(plan, bufs, P, &noop);
    if (rc != RAR_OK || noop)
        return rc;
    if (plan->dtype != RAR_F32 || !w_reps)
        return RAR_EINVAL;
    for (int n = 0; n < plan->N; ++n) {
        rc = check_weights(plan, bufs, w_reps[n]);
        if (rc != RAR_OK)
            return rc;
        const Range a{(uintptr_t)w_reps[n], (uintptr_t)w_reps[n] + (uintptr_t)P * 4};
        for (int m = 0; m < n; ++m)
            if (overlaps(a, {(uintptr_t)w_reps[m], (uintptr_t)w_reps[m] + (uintptr_t)P * 4}))
                return RAR_EINVAL;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (plan->N == 1)
        return run_fused(plan, bufs, w_reps[0], lr, st);
    rc = run_scatter_reduce(plan, bufs, nullptr, w_reps, lr, true, st);
    if (rc != RAR_OK)
        return rc;
    return run_allgather(plan, reinterpret_cast<void *const *>(w_reps), 4, st);
}

extern "C" rar_status rar_allreduce_ring_noalloc(rar_plan_t plan, void *const bufs[], float *w, float lr,
                                                 int64_t P, void *stream)
{
    bool noop;
    rar_status rc = check_exec(plan, bufs, P, &noop);
    if (rc != RAR_OK || noop)
        return rc;
    if (w && (rc = check_weights(plan, bufs, w)) != RAR_OK)
        return rc;
    const bool need_ws = plan->dtype == RAR_BF16 && plan->N > 1;
    if (need_ws && P > RAR_STATIC_WS_ELEMS)
        return RAR_ETOOLARGE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rar_plan_s ring = *plan;  // the plan's table and launch cap, the ring, the static workspace
    ring.algo = RAR_ALGO_RING;
    ring.ws = nullptr;
    if (need_ws) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return hip_failed(e);
        if (st) {
            hipDevice_t sd = cur;
            if ((e = hipStreamGetDevice(st, &sd)) != hipSuccess)
                return hip_failed(e);
            if (sd != cur)
                return RAR_EINVAL;
        }
        if ((e = rar::static_workspace(cur, &ring.ws)) != hipSuccess)
            return hip_failed(e);
    }
    return run_ring(&ring, bufs, w, lr, st);
}

// =============================================================================
// Buckets ([Gibiansky] §Applying allreduce to deep learning)
// =============================================================================

namespace {
struct Segment {
    int tensor;
    int64_t toff, boff, len;
};
}  // namespace

struct rar_buckets_s {
    rar_dtype dtype = RAR_F32;
    int n_tensors = 0;
    int64_t per_bucket = 0;
    int64_t total = 0;              // elements of all tensors
    std::vector<int64_t> numel;     // per tensor
    std::vector<int64_t> start, elems;
    std::vector<std::vector<Segment>> segs;
    int64_t max_elems = 0;
    std::mutex mu;  // guards the plan cache and the workspace
    std::map<std::tuple<int, int64_t, int, int>, rar_plan_t> plans;
    float *ws = nullptr;  // bf16 ring over arenas: binary32 partial sums, `total` floats
    ~rar_buckets_s()
    {
        for (auto &kv : plans)
            rar_plan_destroy(kv.second);
        if (ws)
            (void)hipFree(ws);
    }
};

extern "C" rar_status rar_bucket_plan(int n_tensors, const int64_t numel[], rar_dtype dtype, int64_t bucket_bytes,
                                      rar_buckets_t *out)
{
    if (!out)
        return RAR_EINVAL;
    *out = nullptr;
    if (n_tensors < 0 || (n_tensors > 0 && !numel) || !valid_dtype(dtype))
        return RAR_EINVAL;
    const int64_t B = bucket_bytes / elem_bytes(dtype);
    if (B <= 0)
        return RAR_EINVAL;
    int64_t total = 0;
    for (int t = 0; t < n_tensors; ++t) {
        if (numel[t] < 0 || numel[t] > INT64_MAX - total)
            return RAR_EINVAL;
        total += numel[t];
    }
    if (total / B >= INT32_MAX)  // bucket indices are int
        return RAR_EINVAL;
    return no_throw([&]() -> rar_status {
        std::unique_ptr<rar_buckets_s> b(new rar_buckets_s);
        b->dtype = dtype;
        b->n_tensors = n_tensors;
        b->per_bucket = B;
        if (n_tensors > 0)
            b->numel.assign(numel, numel + n_tensors);
        int64_t stream_pos = 0, fill = 0;
        std::vector<Segment> cur;
        auto close = [&]() {
            b->start.push_back(stream_pos - fill);
            b->elems.push_back(fill);
            b->max_elems = std::max(b->max_elems, fill);
            b->segs.push_back(std::move(cur));
            cur.clear();
            fill = 0;
        };
        for (int t = 0; t < n_tensors; ++t) {
            int64_t done = 0;
            while (done < numel[t]) {
                const int64_t take = std::min(numel[t] - done, B - fill);
                cur.push_back({t, done, fill, take});
                done += take;
                fill += take;
                stream_pos += take;
                if (fill == B)
                    close();
            }
        }
        if (fill > 0)
            close();
        b->total = stream_pos;
        *out = b.release();
        return RAR_OK;
    });
}

extern "C" rar_status rar_bucket_destroy(rar_buckets_t b)
{
    delete b;
    return RAR_OK;
}

extern "C" rar_status rar_bucket_count(rar_buckets_t b, int *n_buckets, int64_t *max_bucket_elems)
{
    if (!b)
        return RAR_EINVAL;
    if (n_buckets)
        *n_buckets = (int)b->segs.size();
    if (max_bucket_elems)
        *max_bucket_elems = b->max_elems;
    return RAR_OK;
}

extern "C" rar_status rar_bucket_info(rar_buckets_t b, int bucket, int64_t *stream_offset, int64_t *elems,
                                      int *n_segments)
{
    if (!b || bucket < 0 || bucket >= (int)b->segs.size())
        return RAR_EINVAL;
    if (stream_offset)
        *stream_offset = b->start[bucket];
    if (elems)
        *elems = b->elems[bucket];
    if (n_segments)
        *n_segments = (int)b->segs[bucket].size();
    return RAR_OK;
}

extern "C" rar_status rar_bucket_segment(rar_buckets_t b, int bucket, int seg, int *tensor, int64_t *tensor_offset,
                                         int64_t *bucket_offset, int64_t *length)
{
    if (!b || bucket < 0 || bucket >= (int)b->segs.size() || seg < 0 || seg >= (int)b->segs[bucket].size())
        return RAR_EINVAL;
    const Segment &s = b->segs[bucket][seg];
    if (tensor)
        *tensor = s.tensor;
    if (tensor_offset)
        *tensor_offset = s.toff;
    if (bucket_offset)
        *bucket_offset = s.boff;
    if (length)
        *length = s.len;
    return RAR_OK;
}

namespace {

rar_status check_bucket_args(rar_buckets_t b, int bucket, int N, void *const tensors[], void *const bucket_bufs[],
                             bool need_bufs = true)
{
    if (!b || bucket < 0 || bucket >= (int)b->segs.size() || N < 1 || N > kMaxRanks || !tensors ||
        (need_bufs && !bucket_bufs))
        return RAR_EINVAL;
    const int es = elem_bytes(b->dtype);
    for (int n = 0; n < N; ++n) {
        if (bucket_bufs && !bucket_bufs[n])
            return RAR_EINVAL;
        if (bucket_bufs && ((uintptr_t)bucket_bufs[n] & 15))
            return RAR_EALIGN;
        for (const Segment &s : b->segs[bucket]) {
            const void *t = tensors[(int64_t)n * b->n_tensors + s.tensor];
            if (!t)
                return RAR_EINVAL;
            if ((uintptr_t)t % es)
                return RAR_EALIGN;
        }
    }
    // the N ranks' copies of a segment must be distinct memory (each rank
    // writes its own copy; shared memory would race)
    Range r[kMaxRanks];
    for (const Segment &s : b->segs[bucket]) {
        for (int n = 0; n < N; ++n) {
            const uintptr_t t = (uintptr_t)tensors[(int64_t)n * b->n_tensors + s.tensor] + (uintptr_t)s.toff * es;
            r[n] = {t, t + (uintptr_t)s.len * es};
        }
        std::sort(r, r + N, [](const Range &a, const Range &c) { return a.lo < c.lo; });
        for (int n = 1; n < N; ++n)
            if (r[n].lo < r[n - 1].hi)
                return RAR_EINVAL;
    }
    if (!bucket_bufs)
        return RAR_OK;
    // the bucket's part of each bucket buffer must overlap neither the other
    // buffers nor any segment copied to or from it (a copy launch would race)
    const uintptr_t kb = (uintptr_t)b->elems[bucket] * es;
    Range bb[kMaxRanks];
    for (int n = 0; n < N; ++n)
        bb[n] = {(uintptr_t)bucket_bufs[n], (uintptr_t)bucket_bufs[n] + kb};
    std::sort(bb, bb + N, [](const Range &a, const Range &c) { return a.lo < c.lo; });
    for (int n = 1; n < N; ++n)
        if (bb[n].lo < bb[n - 1].hi)
            return RAR_EINVAL;
    // sorted and disjoint, so the ends ascend too: the first buffer ending
    // after a segment starts is the only one it can overlap
    for (const Segment &s : b->segs[bucket])
        for (int n = 0; n < N; ++n) {
            const uintptr_t t = (uintptr_t)tensors[(int64_t)n * b->n_tensors + s.tensor] + (uintptr_t)s.toff * es;
            const Range seg{t, t + (uintptr_t)s.len * es};
            const Range *m = std::upper_bound(bb, bb + N, seg.lo, [](uintptr_t x, const Range &a) { return x < a.hi; });
            if (m != bb + N && overlaps(seg, *m))
                return RAR_EINVAL;
        }
    return RAR_OK;
}

bool valid_bucket_call(int N, rar_chunking chunking, rar_algo algo)
{
    return N >= 1 && N <= kMaxRanks &&
           (chunking == RAR_CHUNK_BALANCED || chunking == RAR_CHUNK_CEIL || chunking == RAR_CHUNK_ALIGN16) &&
           (algo == RAR_ALGO_FUSED || algo == RAR_ALGO_RING || algo == RAR_ALGO_NAIVE);
}

// Byte ranges [lo, hi) must be pairwise disjoint (empty ranges are ignored).
bool disjoint(std::vector<Range> &r)
{
    r.erase(std::remove_if(r.begin(), r.end(), [](const Range &x) { return x.hi <= x.lo; }), r.end());
    std::sort(r.begin(), r.end(), [](const Range &a, const Range &c) { return a.lo < c.lo; });
    for (size_t i = 1; i < r.size(); ++i)
        if (r[i].lo < r[i - 1].hi)
            return false;
    return true;
}

// Every tensor of every rank is distinct memory.  Jobs of consecutive
// buckets share a launch, so memory that two tensors share would race.
rar_status check_tensors_disjoint(rar_buckets_t b, int N, void *const tensors[])
{
    const int es = elem_bytes(b->dtype);
    std::vector<Range> r;
    r.reserve((size_t)N * b->n_tensors);
    for (int n = 0; n < N; ++n)
        for (int t = 0; t < b->n_tensors; ++t) {
            const uintptr_t lo = (uintptr_t)tensors[(int64_t)n * b->n_tensors + t];
            if (b->numel[t] > 0 && !lo)
                return RAR_EINVAL;
            r.push_back({lo, lo + (uintptr_t)b->numel[t] * es});
        }
    return disjoint(r) ? RAR_OK : RAR_EINVAL;
}

// Jobs of the grouped bucket kernel, gathered across buckets and launched
// min(kMaxJobs, kMaxJobPtrs / N) at a time.  A launch's grid has one row of
// workgroups per job, as long as its longest job, so jobs under 1 MiB per
// rank (short tensors, bucket ends) gather in a batch of their own and do not
// pad their rows to the length of full chunks.  The jobs are disjoint, so the
// grouping changes no result.
struct JobBatch {
    struct Batch {
        rar::JobsParams jp{};
        int64_t max_len = 0;
    };
    static constexpr int64_t kSmallBytes = 1 << 20;
    rar_dtype dt;
    int N;
    hipStream_t st;
    int per_launch;
    Batch big, small;

    JobBatch(rar_dtype dt_, int N_, hipStream_t st_)
        : dt(dt_), N(N_), st(st_), per_launch(std::min(rar::kMaxJobs, rar::kMaxJobPtrs / N_))
    {
    }

    rar_status flush(Batch &bt)
    {
        if (bt.jp.njobs == 0)
            return RAR_OK;
        hipError_t e = rar::launch_bucket_jobs(dt, N, bt.jp, kDefaultBlocks, bt.max_len, st);
        bt.jp.njobs = 0;
        bt.max_len = 0;
        return hip_status(e);
    }

    rar_status flush()
    {
        rar_status rc = flush(big);
        return rc != RAR_OK ? rc : flush(small);
    }

    // One job of `len` elements whose fold starts at rank c; rank n's first
    // element is at first[n].
    rar_status add(int64_t len, int c, char *const first[])
    {
        if (len <= 0)
            return RAR_OK;
        Batch &bt = len * elem_bytes(dt) < kSmallBytes ? small : big;
        const int j = bt.jp.njobs;
        bool same_align = true;
        for (int n = 0; n < N; ++n) {
            bt.jp.ptr[j * N + n] = first[n];
            same_align &= (((uintptr_t)first[n] ^ (uintptr_t)first[0]) & 15) == 0;
        }
        bt.jp.job[j] = {len, c, same_align ? 1 : 0};
        bt.jp.njobs = j + 1;
        bt.max_len = std::max(bt.max_len, len);
        return bt.jp.njobs == per_launch ? flush(bt) : RAR_OK;
    }
};

// pack (to_bucket) or unpack, in launches of at most kMaxCopyJobs segments
rar_status bucket_copy(rar_buckets_t b, int bucket, int N, void *const tensors[], void *const bucket_bufs[],
                       bool to_bucket, hipStream_t st)
{
    const int es = elem_bytes(b->dtype);
    rar::CopyParams cp{};
    cp.unit = es;
    int64_t max_bytes = 0;
    auto flush = [&]() -> rar_status {
        hipError_t e = rar::launch_copy(cp, kDefaultBlocks, max_bytes, st);
        cp.njobs = 0;
        max_bytes = 0;
        return hip_status(e);
    };
    for (int n = 0; n < N; ++n) {
        for (const Segment &s : b->segs[bucket]) {
            char *t = static_cast<char *>(tensors[(int64_t)n * b->n_tensors + s.tensor]) + s.toff * es;
            char *k = static_cast<char *>(bucket_bufs[n]) + s.boff * es;
            cp.job[cp.njobs++] = to_bucket ? rar::CopyJob{t, k, s.len * es} : rar::CopyJob{k, t, s.len * es};
            max_bytes = std::max(max_bytes, s.len * es);
            if (cp.njobs == rar::kMaxCopyJobs) {
                rar_status rc = flush();
                if (rc != RAR_OK)
                    return rc;
            }
        }
    }
    return cp.njobs ? flush() : RAR_OK;
}

}  // namespace

extern "C" rar_status rar_bucket_pack(rar_buckets_t b, int bucket, int N, void *const tensors[],
                                      void *const bucket_bufs[], void *stream)
{
    rar_status rc = check_bucket_args(b, bucket, N, tensors, bucket_bufs);
    if (rc != RAR_OK)
        return rc;
    return bucket_copy(b, bucket, N, tensors, bucket_bufs, true, static_cast<hipStream_t>(stream));
}

extern "C" rar_status rar_bucket_unpack(rar_buckets_t b, int bucket, int N, void *const bucket_bufs[],
                                        void *const tensors[], void *stream)
{
    rar_status rc = check_bucket_args(b, bucket, N, tensors, bucket_bufs);
    if (rc != RAR_OK)
        return rc;
    return bucket_copy(b, bucket, N, tensors, bucket_bufs, false, static_cast<hipStream_t>(stream));
}

namespace {

// Plans for the distinct bucket sizes, made once and kept with the buckets.
rar_status bucket_plans(rar_buckets_t b, int N, rar_chunking chunking, rar_algo algo,
                        std::vector<rar_plan_t> &plan_of)
{
    const int nb = (int)b->segs.size();
    plan_of.assign(nb, nullptr);
    std::lock_guard<std::mutex> lock(b->mu);
    for (int k = 0; k < nb; ++k) {
        auto key = std::make_tuple(N, b->elems[k], (int)chunking, (int)algo);
        auto it = b->plans.find(key);
        if (it == b->plans.end()) {
            rar_plan_t pl = nullptr;
            rar_status rc = rar_plan(N, b->elems[k], b->dtype, chunking, &pl);
            if (rc == RAR_OK)
                rc = rar_plan_set_algo(pl, algo);
            if (rc != RAR_OK) {
                rar_plan_destroy(pl);
                return rc;
            }
            it = b->plans.emplace(key, pl).first;
        }
        plan_of[k] = it->second;
    }
    return RAR_OK;
}

}  // namespace

namespace {

// Bucket k cut into pieces in the tensors: each segment is cut at the
// bucket's chunk boundaries into pieces with a uniform fold start.  A piece
// that continues the previous one (same chunk, and in every rank it starts
// where the previous one ends: tensors that are views of one flat buffer)
// extends it, so such tensors give the pieces of one flat arena.  Each piece
// goes to sink.add(len, c, first) (first[n]: rank n's first element).
template <class Sink>
rar_status bucket_pieces(rar_buckets_t b, int k, int N, const rar_plan_s *pl, void *const tensors[], Sink &jb)
{
    const int es = elem_bytes(b->dtype);
    char *first[kMaxRanks], *next[kMaxRanks];
    int64_t len = 0;  // pending job: len elements from first[], fold start c
    int c_pending = -1;
    for (const Segment &sg : b->segs[k]) {
        for (int c = 0; c < N; ++c) {
            const int64_t lo = std::max(sg.boff, pl->ct.off[c]);
            const int64_t hi = std::min(sg.boff + sg.len, pl->ct.off[c + 1]);
            if (hi <= lo)
                continue;
            for (int n = 0; n < N; ++n)
                next[n] = static_cast<char *>(tensors[(int64_t)n * b->n_tensors + sg.tensor]) +
                          (sg.toff + (lo - sg.boff)) * es;
            bool extends = len > 0 && c == c_pending;
            for (int n = 0; n < N && extends; ++n)
                extends = next[n] == first[n] + len * es;
            if (extends) {
                len += hi - lo;
                continue;
            }
            if (len > 0) {
                rar_status rc = jb.add(len, c_pending, first);
                if (rc != RAR_OK)
                    return rc;
            }
            std::copy(next, next + N, first);
            len = hi - lo;
            c_pending = c;
        }
    }
    return len > 0 ? jb.add(len, c_pending, first) : RAR_OK;
}

// The ring steps of [Gibiansky] §Scatter-reduce and §Allgather run straight
// on bucket pieces (binary32): at scatter-reduce step s the piece of chunk c
// moves from rank (c+s) mod N to rank (c+s+1) mod N and is added there (the
// last step, at the owner, divides by N); at all-gather step s it moves from
// rank (c+s-1) mod N to rank (c+s) mod N and overwrites.  Pieces are
// gathered until flush(); then each step is one or a few launches over all
// of them (jobs under 1 MiB in launches of their own, so their grid rows are
// not padded to full chunks).  Pieces of different buckets are disjoint
// memory, so sharing launches changes no result.
struct RingPieces {
    int N;
    hipStream_t st;
    std::vector<int64_t> len;
    std::vector<int> chunk;
    std::vector<char *> ptr;  // piece i, rank n: ptr[i*N + n]

    RingPieces(int N_, hipStream_t st_) : N(N_), st(st_) {}

    rar_status add(int64_t n, int c, char *const first[])
    {
        if (n <= 0)
            return RAR_OK;
        len.push_back(n);
        chunk.push_back(c);
        ptr.insert(ptr.end(), first, first + N);
        return RAR_OK;
    }

    static bool small(int64_t n) { return n * 4 < JobBatch::kSmallBytes; }

    rar_status scatter_reduce_step(int s, bool last)
    {
        for (int pass = 0; pass < 2; ++pass) {  // big pieces, then small ones
            rar::StepJobsParams jp{};
            jp.N = N;
            int64_t mx = 0;
            for (size_t i = 0; i < len.size(); ++i) {
                if (small(len[i]) != (pass == 1))
                    continue;
                const int c = chunk[i];
                jp.job[jp.njobs++] = {reinterpret_cast<const float *>(ptr[i * N + (c + s) % N]),
                                      reinterpret_cast<float *>(ptr[i * N + (c + s + 1) % N]), len[i]};
                mx = std::max(mx, len[i]);
                if (jp.njobs == rar::kMaxStepJobs) {
                    hipError_t e = rar::launch_sr_jobs(jp, last, mx, st);
                    if (e != hipSuccess)
                        return RAR_EHIP;
                    jp.njobs = 0;
                    mx = 0;
                }
            }
            if (jp.njobs && rar::launch_sr_jobs(jp, last, mx, st) != hipSuccess)
                return RAR_EHIP;
        }
        return RAR_OK;
    }

    rar_status allgather_step(int s)
    {
        for (int pass = 0; pass < 2; ++pass) {
            rar::CopyParams cp{};
            cp.unit = 4;
            int64_t mx = 0;
            for (size_t i = 0; i < len.size(); ++i) {
                if (small(len[i]) != (pass == 1))
                    continue;
                const int c = chunk[i];
                cp.job[cp.njobs++] = {ptr[i * N + (c + s - 1 + N) % N], ptr[i * N + (c + s) % N], len[i] * 4};
                mx = std::max(mx, len[i] * 4);
                if (cp.njobs == rar::kMaxCopyJobs) {
                    if (rar::launch_copy(cp, kDefaultBlocks, mx, st) != hipSuccess)
                        return RAR_EHIP;
                    cp.njobs = 0;
                    mx = 0;
                }
            }
            if (cp.njobs && rar::launch_copy(cp, kDefaultBlocks, mx, st) != hipSuccess)
                return RAR_EHIP;
        }
        return RAR_OK;
    }

    rar_status flush()
    {
        rar_status rc = RAR_OK;
        for (int s = 0; s < N - 1 && rc == RAR_OK; ++s)
            rc = scatter_reduce_step(s, s == N - 2);
        for (int s = 0; s < N - 1 && rc == RAR_OK; ++s)
            rc = allgather_step(s);
        len.clear();
        chunk.clear();
        ptr.clear();
        return rc;
    }
};

// Buckets k0 .. k1-1 of per-rank arenas (bucket k of rank n starts at element
// start[k] of base[n]): the fused pass in one launch, or each ring step in one
// launch, over every chunk of every bucket in the range (a launch holds up to
// 65535 rows of one chunk each, so very long ranges take a few).  Every bucket
// but the plan's last holds B elements, so two chunk tables describe them all.
rar_status arena_run(rar_buckets_t b, int N, const std::vector<rar_plan_t> &plan_of, char *const base[], int k0,
                     int k1, rar_algo algo, hipStream_t st)
{
    const int es = elem_bytes(b->dtype);
    const int per = 65535 / N;
    float *ws = nullptr;
    if (algo == RAR_ALGO_RING && b->dtype == RAR_BF16 && k1 > k0) {
        // the binary32 partial sums of a bf16 ring: allocated on first use,
        // kept with the buckets
        std::lock_guard<std::mutex> lock(b->mu);
        if (!b->ws) {
            void *p = nullptr;
            const hipError_t e = hipMalloc(&p, (size_t)b->total * sizeof(float));
            if (e != hipSuccess)
                return hip_failed(e);
            b->ws = static_cast<float *>(p);
        }
        ws = b->ws;
    }
    std::vector<rar::ArenaParams> launches;
    std::vector<int64_t> max_chunk;
    for (int a = k0; a < k1; a += per) {
        const int e = std::min(k1, a + per);
        rar::ArenaParams p{};
        p.N = N;
        p.B = b->per_bucket;
        p.nb = e - a;
        for (int n = 0; n < N; ++n)
            p.base[n] = base[n] + b->start[a] * es;
        const rar_plan_s *first = plan_of[a], *lastp = plan_of[e - 1];
        p.full = first->ct;
        p.last = lastp->ct;
        p.last_partial = b->elems[e - 1] != b->per_bucket ? 1 : 0;
        p.ws = ws ? ws + b->start[a] : nullptr;
        launches.push_back(p);
        max_chunk.push_back(std::max(first->max_chunk, lastp->max_chunk));
    }
    auto launch = [&](rar::ArenaOp op, int s) -> rar_status {
        for (size_t i = 0; i < launches.size(); ++i) {
            launches[i].s = s;
            if (rar::launch_arena(b->dtype, op, launches[i], max_chunk[i], st) != hipSuccess)
                return RAR_EHIP;
        }
        return RAR_OK;
    };
    if (algo == RAR_ALGO_FUSED)
        return launch(rar::kArenaFused, 0);
    rar_status rc = RAR_OK;
    for (int s = 0; s < N - 1 && rc == RAR_OK; ++s) {
        const bool first = s == 0, last = s == N - 2;
        rc = launch(first && last ? rar::kArenaScatterReduceFirstLast
                    : first       ? rar::kArenaScatterReduceFirst
                    : last        ? rar::kArenaScatterReduceLast
                                  : rar::kArenaScatterReduce,
                    s);
    }
    for (int s = 0; s < N - 1 && rc == RAR_OK; ++s)
        rc = launch(rar::kArenaAllgather, s);
    return rc;
}

// Tensor lists that are per-rank arenas: every rank's tensors lie end to end
// in the plan's order (views of one flat buffer per rank, the usual layout of
// gradient buckets) from a 16-byte aligned start, and bucket starts are 16-byte
// aligned.  base[n] receives rank n's start.
bool tensors_form_arenas(rar_buckets_t b, int N, void *const tensors[], char *base[])
{
    const int es = elem_bytes(b->dtype);
    if ((b->per_bucket * es) % 16 != 0)
        return false;
    for (int n = 0; n < N; ++n) {
        // addresses as integers: the call is validated only afterwards, so a
        // pointer here may be null
        uintptr_t b0 = 0;
        int64_t cum = 0;
        for (int t = 0; t < b->n_tensors; ++t) {
            if (b->numel[t] > 0) {
                const uintptr_t p = reinterpret_cast<uintptr_t>(tensors[(int64_t)n * b->n_tensors + t]);
                if (!p)
                    return false;
                if (!b0)
                    b0 = p;  // every earlier tensor is empty: this one starts the arena
                if (p != b0 + (uintptr_t)cum * es)
                    return false;
            }
            cum += b->numel[t];
        }
        if (!b0 || (b0 & 15))
            return false;
        base[n] = reinterpret_cast<char *>(b0);
    }
    return true;
}

// Buckets whose ring steps run on their pieces in place: binary32 at N >= 2
// (bf16 keeps its partial sums in a plan's workspace and goes through bucket
// buffers; one rank has no transfers).
bool ring_on_pieces(rar_dtype dt, int N, rar_algo algo) { return algo == RAR_ALGO_RING && dt == RAR_F32 && N >= 2; }

}  // namespace

extern "C" rar_status rar_bucket_allreduce_mean(rar_buckets_t b, int N, rar_chunking chunking, rar_algo algo,
                                                void *const tensors[], void *const bucket_bufs[], void *stream)
{
    return no_throw([&]() -> rar_status {
        if (!b || !valid_bucket_call(N, chunking, algo))
            return RAR_EINVAL;
        const int nb = (int)b->segs.size();
        // host arithmetic on the given addresses only; validated below
        char *base[kMaxRanks];
        const bool arenas = tensors && tensors_form_arenas(b, N, tensors, base);
        const bool ring_direct = ring_on_pieces(b->dtype, N, algo) || (algo == RAR_ALGO_RING && N >= 2 && arenas);
        const bool direct = (algo == RAR_ALGO_FUSED && rar::bucket_jobs_supported(N)) || ring_direct;
        for (int k = 0; k < nb; ++k) {
            rar_status rc = check_bucket_args(b, k, N, tensors, bucket_bufs, !direct);
            if (rc != RAR_OK)
                return rc;
        }
        std::vector<rar_plan_t> plan_of;
        rar_status rc = bucket_plans(b, N, chunking, algo, plan_of);
        if (rc != RAR_OK)
            return rc;
        hipStream_t st = static_cast<hipStream_t>(stream);
        if (direct) {
            rc = check_tensors_disjoint(b, N, tensors);
            if (rc != RAR_OK)
                return rc;
            if (arenas)
                return arena_run(b, N, plan_of, base, 0, nb, ring_direct ? RAR_ALGO_RING : RAR_ALGO_FUSED, st);
            if (ring_direct) {
                RingPieces rp(N, st);
                for (int k = 0; k < nb && rc == RAR_OK; ++k)
                    rc = bucket_pieces(b, k, N, plan_of[k], tensors, rp);
                return rc != RAR_OK ? rc : rp.flush();
            }
            JobBatch jb(b->dtype, N, st);
            for (int k = 0; k < nb; ++k) {
                rc = bucket_pieces(b, k, N, plan_of[k], tensors, jb);
                if (rc != RAR_OK)
                    return rc;
            }
            return jb.flush();
        }
        for (int k = 0; k < nb; ++k) {
            rc = bucket_copy(b, k, N, tensors, bucket_bufs, true, st);
            if (rc == RAR_OK)
                rc = rar_allreduce_mean(plan_of[k], bucket_bufs, b->elems[k], stream);
            if (rc == RAR_OK)
                rc = bucket_copy(b, k, N, tensors, bucket_bufs, false, st);
            if (rc != RAR_OK)
                return rc;
        }
        return RAR_OK;
    });
}

extern "C" rar_status rar_bucket_allreduce_arena(rar_buckets_t b, int N, rar_chunking chunking, rar_algo algo,
                                                 void *const arenas[], void *const ready_events[], void *stream)
{
    return no_throw([&]() -> rar_status {
        if (!b || !arenas || !valid_bucket_call(N, chunking, algo))
            return RAR_EINVAL;
        const int es = elem_bytes(b->dtype);
        const int nb = (int)b->segs.size();
        for (int n = 0; n < N; ++n) {
            if (!arenas[n])
                return RAR_EINVAL;
            if ((uintptr_t)arenas[n] & 15)
                return RAR_EALIGN;
        }
        for (int k = 0; k < nb; ++k)
            if ((b->start[k] * es) & 15)
                return RAR_EALIGN;
        std::vector<Range> ar;
        for (int n = 0; n < N; ++n)
            ar.push_back({(uintptr_t)arenas[n], (uintptr_t)arenas[n] + (uintptr_t)b->total * es});
        if (!disjoint(ar))
            return RAR_EINVAL;
        std::vector<rar_plan_t> plan_of;
        rar_status rc = bucket_plans(b, N, chunking, algo, plan_of);
        if (rc != RAR_OK)
            return rc;
        hipStream_t st = static_cast<hipStream_t>(stream);
        if ((algo == RAR_ALGO_FUSED && rar::bucket_jobs_supported(N)) || (algo == RAR_ALGO_RING && N >= 2)) {
            // the buckets between two ready events share the launches
            char *base[kMaxRanks];
            for (int n = 0; n < N; ++n)
                base[n] = static_cast<char *>(arenas[n]);
            int k0 = 0;
            for (int k = 0; k < nb; ++k) {
                if (ready_events && ready_events[k]) {
                    rc = arena_run(b, N, plan_of, base, k0, k, algo, st);
                    if (rc != RAR_OK)
                        return rc;
                    const hipError_t e = hipStreamWaitEvent(st, static_cast<hipEvent_t>(ready_events[k]), 0);
                    if (e != hipSuccess)
                        return hip_failed(e);
                    k0 = k;
                }
            }
            return arena_run(b, N, plan_of, base, k0, nb, algo, st);
        }
        void *slice[kMaxRanks];
        for (int k = 0; k < nb; ++k) {
            if (ready_events && ready_events[k]) {
                const hipError_t e = hipStreamWaitEvent(st, static_cast<hipEvent_t>(ready_events[k]), 0);
                if (e != hipSuccess)
                    return hip_failed(e);
            }
            for (int n = 0; n < N; ++n)
                slice[n] = static_cast<char *>(arenas[n]) + b->start[k] * es;
            rc = rar_allreduce_mean(plan_of[k], slice, b->elems[k], stream);
            if (rc != RAR_OK)
                return rc;
        }
        return RAR_OK;
    });
}

// =============================================================================

extern "C" const char *rar_strerror(rar_status s)
{
    switch (s) {
    case RAR_OK: return "success";
    case RAR_EINVAL: return "invalid argument";
    case RAR_EMISMATCH: return "element count differs from the plan";
    case RAR_EALIGN: return "device pointer not 16-byte aligned";
    case RAR_ENOMEM: return "out of memory";
    case RAR_EHIP: return "HIP runtime error";
    case RAR_ETOOLARGE: return "element count exceeds the static workspace";
    }
    return "unknown status";
}

extern "C" int rar_version(void) { return 600; }  // 0.6.0: rar_rank_stride_candidate, wider stride search
