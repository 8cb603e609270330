// rar_internal.h -- declarations shared by the host code (rar_host.cpp) and the
// kernels (rar_kernels.hip) of librar.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rar.h"

namespace rar {

constexpr int kMaxRanks = RAR_MAX_RANKS;
constexpr int kThreads = 256;   // workgroup size of every kernel: four 64-wide waves
constexpr int kMaxCopyJobs = 128;

// Chunk table: chunk c is [off[c], off[c+1]).  Passed to kernels by value in the
// kernel-argument segment, so a wave-uniform index becomes a scalar load.
struct ChunkTable {
    int64_t off[kMaxRanks + 1];
};

struct RankPtrs {
    void *p[kMaxRanks];
};

// Fused single pass: every rank read once, every rank written once.
struct FusedParams {
    RankPtrs bufs;
    ChunkTable ct;
    float *w;     // nullptr: mean only
    float lr;
    int N;
};

// One ring step, all N chunk transfers of the step in one launch.
struct StepParams {
    RankPtrs bufs;
    RankPtrs wreps;  // per-rank weight replicas (sharded update), else unused
    ChunkTable ct;
    float *w;        // shared weights (nullptr: none)
    float *ws;       // binary32 chunk-indexed workspace (bf16 ring), else nullptr
    float lr;
    int N;
    int s;           // step index within its phase
    int sharded;     // 1: the owner updates wreps[owner] instead of w
};

struct CopyJob {
    const void *src;
    void *dst;
    int64_t nbytes;
};

struct CopyParams {
    CopyJob job[kMaxCopyJobs];
    int njobs;
    int unit;  // element size in bytes (2 or 4) for unaligned remainders
};

// One job of a bucket reduced straight from the tensors: `len` elements whose
// fold starts at rank c; vec_ok == 0 when the ranks' pointers differ in their
// 16-byte alignment (scalar path).
struct JobDesc {
    int64_t len;
    int32_t c;
    int32_t vec_ok;
};

constexpr int kMaxJobs = 48;
constexpr int kMaxJobPtrs = 320;

struct JobsParams {
    void *ptr[kMaxJobPtrs];  // job j, rank r: ptr[j*N + r]
    JobDesc job[kMaxJobs];
    int njobs;
};

// Ring steps straight on bucket pieces: one transfer per piece per step, the
// receiver's piece += the sender's (binary32), divided by N on the last
// scatter-reduce step.
struct StepJob {
    const float *src;
    float *dst;
    int64_t len;  // elements
};

constexpr int kMaxStepJobs = 128;

struct StepJobsParams {
    StepJob job[kMaxStepJobs];
    int njobs;
    int N;
};

// Consecutive buckets of per-rank arenas: rank n's bucket k starts at element
// k*B of base[n], and the piece of bucket k, chunk c is elements
// [k*B + off[c], k*B + off[c+1]) in every rank, off from `full`, or from `last`
// for the final bucket when last_partial.  Workgroup row y is bucket y / N,
// chunk y % N.
struct ArenaParams {
    void *base[kMaxRanks];
    ChunkTable full;
    ChunkTable last;
    int64_t B;
    int nb;
    int last_partial;
    int N;
    int s;      // ring step within its phase
    float *ws;  // bf16 ring: binary32 partial sums, indexed like the arenas' elements
};

// The first scatter-reduce step differs only for bf16 (partial sums start in ws).
enum ArenaOp {
    kArenaFused = 0,
    kArenaScatterReduce = 1,
    kArenaScatterReduceLast = 2,
    kArenaAllgather = 3,
    kArenaScatterReduceFirst = 4,
    kArenaScatterReduceFirstLast = 5
};

// Single reducer (prior art): rank 0 accumulates rank `src`.
struct PairParams {
    RankPtrs bufs;
    float *w;
    float lr;
    int N;
    int src;
    int64_t P;
};

// ---- launchers (rar_kernels.hip); each returns hipSuccess or the launch error
hipError_t launch_fused(rar_dtype dt, const FusedParams &p, int max_blocks, int64_t max_chunk,
                        hipStream_t st);
hipError_t launch_sr_step(rar_dtype dt, const StepParams &p, bool first, bool last, bool sgd,
                          int max_blocks, int64_t max_chunk, hipStream_t st);
hipError_t launch_copy(const CopyParams &p, int max_blocks, int64_t max_job_bytes, hipStream_t st);
hipError_t launch_pair_add(const PairParams &p, bool last, bool sgd, int max_blocks, hipStream_t st);
hipError_t launch_sr_jobs(const StepJobsParams &p, bool last, int64_t max_len, hipStream_t st);
// op kArenaFused: dt either, N with a grouped kernel (bucket_jobs_supported);
// the ring ops: any N >= 2, bf16 with p.ws set.
hipError_t launch_arena(rar_dtype dt, ArenaOp op, const ArenaParams &p, int64_t max_chunk, hipStream_t st);
// The binary32 workspace held in the library's static device array: its
// address on `device`, which must be the current device (looked up on the
// first call for that device, then kept).
constexpr int kMaxDevices = 64;
hipError_t static_workspace(int device, float **ptr);
// Rank counts with a bucket-jobs kernel (others use pack, reduce, unpack).
bool bucket_jobs_supported(int N);
hipError_t launch_bucket_jobs(rar_dtype dt, int N, const JobsParams &p, int max_blocks, int64_t max_len,
                              hipStream_t st);

}  // namespace rar
