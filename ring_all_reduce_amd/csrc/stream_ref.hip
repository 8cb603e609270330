// stream_ref.hip -- reference stream kernels for the benchmark (libstream_ref.so).
//
// Measurement only: nothing here is a step of the all-reduce, and librar.so
// neither links nor calls it.  The kernels move data in exactly the access
// pattern of the grouped fused pass -- G groups of 256 lanes per workgroup,
// one 16-byte vector per lane per rank, one tile per workgroup, group g
// owning a run of ceil(N/G) ranks and the last group also the weight stream
// -- without its fold, division or update.  Timed over the same buffers as
// the fused pass, they give the rate HBM sustains for that pattern:
//   mode 0  move in place: every stream read, then written back unchanged
//           (the fused pass's bytes and streams exactly);
//   mode 1  write only (no reads);
//   mode 2  read only (the loaded data decide whether anything is stored, to a
//           4 KiB sink, so the loads are not removed);
//   mode 3  a plain copy of rank 0 into rank 1 (one vector per lane, one tile
//           per workgroup, no job table): the 1 -> 1 streaming reference;
//   mode 4  move in place as mode 0, for 10 binary32 ranks and the weights
//           only, with the eleven pointers in one table and each lane
//           checking its index per access.  The same bytes, streams, groups
//           and order as mode 0; only the compiled code differs: here each
//           wave gets two of its stores out at a time, and that form moved
//           these streams fastest of the movers measured.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLanes = 256;
constexpr int kMaxRanks = 64;

struct SrefParams {
    void *rank[kMaxRanks];
    u32x4 *w;        // weight stream: WV vectors per lane-vector (nullptr: none)
    u32x4 *sink;     // mode 2: 256 vectors
    int64_t vecs;    // 16-byte vectors per rank
    uint32_t key;    // 0 at run time; XORed into what mode 0 writes back, so the
                     // compiler cannot drop a store of the value just loaded
};

template <typename V>
__device__ __forceinline__ V ld(const V *p)
{
    return __builtin_nontemporal_load(p);
}

template <typename V>
__device__ __forceinline__ void st(V *p, V v)
{
    __builtin_nontemporal_store(v, p);
}

template <int NR, int G, int WV, int MODE>
__global__ __launch_bounds__(kLanes *G) void sref_streams(SrefParams p)
{
    constexpr int PER = (NR + G - 1) / G;
    const int g = threadIdx.x / kLanes;
    const int lane = threadIdx.x % kLanes;
    const int k0 = g * PER;
    const int cnt = k0 >= NR ? 0 : (NR - k0 < PER ? NR - k0 : PER);
    const int64_t v = (int64_t)blockIdx.x * kLanes + lane;
    if (v >= p.vecs)
        return;  // no barrier follows
    const bool has_w = WV > 0 && g == G - 1;
    u32x4 x[PER];
    u32x4 wv[WV > 0 ? WV : 1];
    if (MODE != 1) {
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (j < cnt)
                x[j] = ld(static_cast<const u32x4 *>(p.rank[k0 + j]) + v);
        if (has_w) {
#pragma unroll
            for (int i = 0; i < WV; ++i)
                wv[i] = ld(p.w + WV * v + i);
        }
    }
    if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (j < cnt)
                st(static_cast<u32x4 *>(p.rank[k0 + j]) + v, x[j] ^ p.key);
        if (has_w) {
#pragma unroll
            for (int i = 0; i < WV; ++i)
                st(p.w + WV * v + i, wv[i] ^ p.key);
        }
    } else if (MODE == 1) {
        const u32x4 c = {(uint32_t)lane, (uint32_t)g, 0u, 0u};
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (j < cnt)
                st(static_cast<u32x4 *>(p.rank[k0 + j]) + v, c);
        if (has_w) {
#pragma unroll
            for (int i = 0; i < WV; ++i)
                st(p.w + WV * v + i, c);
        }
    } else {
        u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (j < cnt)
                acc ^= x[j];
        if (has_w) {
#pragma unroll
            for (int i = 0; i < WV; ++i)
                acc ^= wv[i];
        }
        if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0xf39cc060u && acc.w == 0x5cedc834u)
            p.sink[lane] = acc;
    }
}

// Mode 4: NS streams in one pointer table (the ranks, then w), stream s in
// group s / PER, one vector per lane and stream.
struct TableParams {
    void *s[16];
    int64_t vecs;
    uint32_t key;  // 0 at run time, as in SrefParams
};

template <int NS, int G>
__global__ __launch_bounds__(kLanes *G) void sref_table_move(TableParams p)
{
    constexpr int PER = (NS + G - 1) / G;
    const int g = threadIdx.x / kLanes, lane = threadIdx.x % kLanes;
    const int64_t i = (int64_t)blockIdx.x * kLanes + lane;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (g * PER + j < NS)
            cnt = j + 1;
    u32x4 x[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (j < cnt && i < p.vecs)
            x[j] = ld(static_cast<const u32x4 *>(p.s[g * PER + j]) + i);
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (j < cnt && i < p.vecs)
            st(static_cast<u32x4 *>(p.s[g * PER + j]) + i, x[j] ^ p.key);
}

__global__ __launch_bounds__(kLanes) void sref_copy(SrefParams p)
{
    const int64_t v = (int64_t)blockIdx.x * kLanes + threadIdx.x;
    if (v < p.vecs)
        st(static_cast<u32x4 *>(p.rank[1]) + v, ld(static_cast<const u32x4 *>(p.rank[0]) + v));
}

template <int NR, int G, int WV>
hipError_t launch(int mode, const SrefParams &p, hipStream_t st)
{
    const dim3 grid((unsigned)((p.vecs + kLanes - 1) / kLanes)), block(kLanes * G);
    switch (mode) {
    case 0: hipLaunchKernelGGL((sref_streams<NR, G, WV, 0>), grid, block, 0, st, p); break;
    case 1: hipLaunchKernelGGL((sref_streams<NR, G, WV, 1>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((sref_streams<NR, G, WV, 2>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
}

}  // namespace

// mode: 0 move in place, 1 write only, 2 read only, 3 copy rank 0 into rank 1,
// 4 move in place from one pointer table.
// ranks: n_ranks device pointers of `vecs` 16-byte vectors each; w: w_vpl *
// vecs vectors (w_vpl 1 for binary32 ranks, 2 for bf16 ranks, 0 for no weight
// stream); sink: 4 KiB, needed by mode 2.  Shapes: (n_ranks, groups, w_vpl) in
// {(10,4,1), (10,1,1), (40,4,2), (8,4,0), (1,1,0)}, (2,1,0) for mode 3 (the
// two ranks must not overlap), and (10,4,1) only for mode 4.  Returns 0, -1
// for bad arguments, -5 if the launch failed.
extern "C" int sref_run(int mode, int n_ranks, void *const ranks[], void *w, int w_vpl, int64_t vecs, int groups,
                        void *sink, void *stream)
{
    if (mode < 0 || mode > 4 || n_ranks < 1 || n_ranks > kMaxRanks || !ranks || vecs < 0 ||
        (vecs > 0 && (vecs + kLanes - 1) / kLanes > 0x7fffffff))
        return -1;
    if ((w_vpl > 0) != (w != nullptr) || (mode == 2 && !sink))
        return -1;
    SrefParams p{};
    for (int n = 0; n < n_ranks; ++n) {
        if (!ranks[n] || ((uintptr_t)ranks[n] & 15))
            return -1;
        p.rank[n] = ranks[n];
    }
    if (((uintptr_t)w & 15) || ((uintptr_t)sink & 15))
        return -1;
    p.w = static_cast<u32x4 *>(w);
    p.sink = static_cast<u32x4 *>(sink);
    p.vecs = vecs;
    if (vecs == 0)
        return 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (mode == 3) {
        const uintptr_t a = (uintptr_t)ranks[0], b = (uintptr_t)ranks[1], bytes = (uintptr_t)vecs * 16;
        if (n_ranks != 2 || groups != 1 || w_vpl != 0 || (a < b + bytes && b < a + bytes))
            return -1;
        hipLaunchKernelGGL(sref_copy, dim3((unsigned)((vecs + kLanes - 1) / kLanes)), dim3(kLanes), 0, st, p);
        e = hipGetLastError();
    } else if (mode == 4) {
        if (n_ranks != 10 || groups != 4 || w_vpl != 1)
            return -1;
        TableParams t{};
        for (int n = 0; n < 10; ++n)
            t.s[n] = ranks[n];
        t.s[10] = w;
        t.vecs = vecs;
        hipLaunchKernelGGL((sref_table_move<11, 4>), dim3((unsigned)((vecs + kLanes - 1) / kLanes)),
                           dim3(kLanes * 4), 0, st, t);
        e = hipGetLastError();
    } else if (n_ranks == 10 && groups == 4 && w_vpl == 1)
        e = launch<10, 4, 1>(mode, p, st);
    else if (n_ranks == 10 && groups == 1 && w_vpl == 1)
        e = launch<10, 1, 1>(mode, p, st);
    else if (n_ranks == 40 && groups == 4 && w_vpl == 2)
        e = launch<40, 4, 2>(mode, p, st);
    else if (n_ranks == 8 && groups == 4 && w_vpl == 0)
        e = launch<8, 4, 0>(mode, p, st);
    else if (n_ranks == 1 && groups == 1 && w_vpl == 0)
        e = launch<1, 1, 0>(mode, p, st);
    else
        return -1;
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return -5;
    }
    return 0;
}
