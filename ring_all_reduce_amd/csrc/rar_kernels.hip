// rar_kernels.hip -- CDNA4 (gfx950) kernels of the ring all-reduce-mean + SGD.
//
// Sources: [Gibiansky] "Bringing HPC Techniques to Deep Learning" (A. Gibiansky,
// Baidu SVAIL), sections "Ring allreduce", "Scatter-reduce", "Allgather",
// "Allreduce communication cost"; [TrainMGPU] "[AI System] Training With
// Multiple GPUs", section "Training Process".
//
// All N logical ranks live in one device's HBM, so a ring "transfer" from rank
// n to rank n+1 is a read of rank n's buffer and a write of rank n+1's.  Every
// kernel here is a streaming pass bound by HBM bandwidth (well under one flop
// per byte): there is no contraction and so no MFMA.  What matters is that
// every byte moves once in 16-byte (dwordx4) accesses that coalesce into whole
// cache lines, with enough loads in flight per CU to cover HBM latency, and
// that nothing is re-read.
//
// Work decomposition, shared by every kernel: blockIdx.y selects a job (a
// chunk of the chunk table, a bucket piece, a copy segment, or -- for buckets
// in per-rank arenas -- bucket y / N and its chunk y % N); blockIdx.x and a
// grid-stride loop walk that job's element range.  The body of the range starts on a
// 128-byte cache line and is processed in tiles of kThreads*VPT 16-byte
// vectors, lane-contiguous so that one wave instruction touches 1 KiB of
// consecutive memory and each tile covers whole lines (no line is fetched or
// written by two workgroups).  The elements before that first line (the head)
// and the at most VEC-1 after the last whole vector (the tail) go through a
// scalar path on block 0's first lanes.  Chunk boundaries need not be aligned
// at all (a balanced cut of P = 1,000,003 over 4 ranks puts them at 250,001
// and 500,002), so the per-chunk span keeps a dwordx4 access from ever
// straddling two chunks whose sums start at different ranks.
//
// Numerics, identical in every kernel: binary32 adds in ring order starting at
// the chunk's own rank, one IEEE division by N, SGD as w - (lr*m) with both
// operations rounded (contraction is off, see the pragma), subnormals kept.
#include <mutex>
#include <type_traits>

#include <hip/hip_bf16.h>

#include "rar_internal.h"

#pragma clang fp contract(off)

namespace rar {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming accesses: the data are touched once per call, so keep them from
// displacing other lines in L2 and the Infinity Cache.
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

__device__ __forceinline__ int next_rank(int r, int N)
{
    return (r + 1 == N) ? 0 : r + 1;
}

// ---------------------------------------------------------------------------
// bfloat16: the upper 16 bits of a binary32 pattern.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_one(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest bfloat16, ties to the even pattern; NaN keeps its sign and
// leading payload and gets the quiet bit.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction in the packed helpers
// below).  Checked on the device against the integer form of the same rule
// (add 0x7fff plus the lowest kept bit, keep the upper half; NaN: upper half
// with the quiet bit set) over all 2^32 binary32 patterns, NaN included: no
// difference.  The 40-rank bf16 pass runs 1.6% faster than with the integer
// form.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    return __bfloat16_as_ushort(__float2bfloat16(f));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 widen4(u32x2 u)
{
    return f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
}

__device__ __forceinline__ u32x2 narrow4(f32x4 a)
{
    return u32x2{bf16_rne(a.x) | (bf16_rne(a.y) << 16), bf16_rne(a.z) | (bf16_rne(a.w) << 16)};
}

__device__ __forceinline__ void widen8(u32x4 u, f32x4 &a, f32x4 &b)
{
    a = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
    b = f32x4{bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
}

__device__ __forceinline__ u32x4 narrow8(f32x4 a, f32x4 b)
{
    return u32x4{bf16_rne(a.x) | (bf16_rne(a.y) << 16), bf16_rne(a.z) | (bf16_rne(a.w) << 16),
                 bf16_rne(b.x) | (bf16_rne(b.y) << 16), bf16_rne(b.z) | (bf16_rne(b.w) << 16)};
}

// ---------------------------------------------------------------------------
// Span driver
// ---------------------------------------------------------------------------

// Walk elements [e0, e1) of one job: scalar head (up to the first index on a
// 128-byte line) and tail (after the last whole 16-byte group) on block 0,
// then the body in tiles (grid-stride over blockIdx.x).  VEC = elements per
// 16 bytes.  elem(e) handles one element; tile(FULL, a0, v0, nvec) handles
// vectors v0 .. v0+kThreads*VPT-1 of the body that starts at element a0
// (lane-contiguous), bounds-checked against nvec unless FULL.
template <int VEC, int VPT, class ElemF, class TileF>
__device__ __forceinline__ void run_span(int64_t e0, int64_t e1, ElemF &&elem, TileF &&tile)
{
    if (e1 <= e0)
        return;
    // the body starts at an element index that is a multiple of one 128-byte
    // line (buffers are allocations, so index and address alignment agree),
    // so no line is shared by two workgroups' tiles
    constexpr int64_t LINE = 8 * VEC;
    int64_t h = (LINE - e0 % LINE) % LINE;
    if (h > e1 - e0)
        h = e1 - e0;
    const int64_t a0 = e0 + h;
    const int64_t a1 = a0 + (e1 - a0) / VEC * VEC;
    if (blockIdx.x == 0) {
        const int t = threadIdx.x;
        if (t < LINE) {
            if (t < h)
                elem(e0 + t);
        } else if (t - LINE < e1 - a1) {
            elem(a1 + (t - LINE));
        }
    }
    const int64_t nvec = (a1 - a0) / VEC;
    constexpr int64_t TV = (int64_t)kThreads * VPT;
    const int64_t ntiles = (nvec + TV - 1) / TV;
    for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const int64_t v0 = t * TV;
        if (v0 + TV <= nvec)
            tile(std::true_type{}, a0, v0, nvec);
        else
            tile(std::false_type{}, a0, v0, nvec);
    }
}

template <int VPT, bool FULL>
__device__ __forceinline__ void lane_vectors(int64_t v0, int64_t nvec, int64_t (&vi)[VPT], bool (&ok)[VPT])
{
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        vi[j] = v0 + (int64_t)j * kThreads + threadIdx.x;
        ok[j] = FULL || vi[j] < nvec;
    }
}

template <typename V, typename T>
__device__ __forceinline__ V *vec_at(void *base, int64_t a0)
{
    return reinterpret_cast<V *>(static_cast<T *>(base) + a0);
}

// ---------------------------------------------------------------------------
// Fused single pass, binary32.
// ---------------------------------------------------------------------------
//
// Chunk c = blockIdx.y.  Each lane loads its vectors from ranks c, c+1, ...,
// c+N-1 (mod N) -- the order in which the scatter-reduce of [Gibiansky] folds
// chunk c -- adds them in that order, divides by N, stores the mean into all
// N buffers and, with SGD, updates w.  N compile-time (NT > 0) lets all N-1
// loads of a tile be in flight before the first add; NT == 0 takes N from the
// arguments and keeps KB loads in flight.

template <int NT, int VPT, bool SGD>
__global__ __launch_bounds__(kThreads) void rar_fused_f32(FusedParams p)
{
    const int N = NT > 0 ? NT : p.N;
    const int c = blockIdx.y;
    constexpr int KB = NT > 0 ? (NT > 1 ? NT - 1 : 1) : 8;

    auto elem = [&](int64_t e) {
        float acc = static_cast<const float *>(p.bufs.p[c])[e];
        int r = c;
        for (int k = 1; k < N; ++k) {
            r = next_rank(r, N);
            acc = acc + static_cast<const float *>(p.bufs.p[r])[e];
        }
        const float m = acc / (float)N;
        for (int n = 0; n < N; ++n)
            static_cast<float *>(p.bufs.p[n])[e] = m;
        if (SGD) {
            const float step = p.lr * m;
            p.w[e] = p.w[e] - step;
        }
    };

    auto tile = [&](auto full, int64_t a0, int64_t v0, int64_t nvec) {
        constexpr bool FULL = decltype(full)::value;
        int64_t vi[VPT];
        bool ok[VPT];
        lane_vectors<VPT, FULL>(v0, nvec, vi, ok);
        f32x4 acc[VPT];
        {
            const f32x4 *src = vec_at<const f32x4, const float>(p.bufs.p[c], a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                if (ok[j])
                    acc[j] = ld(src + vi[j]);
        }
        int r = c;
        for (int k = 1; k < N; k += KB) {
            f32x4 x[KB][VPT];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                if (NT > 0 || k + kk < N) {
                    r = next_rank(r, N);
                    const f32x4 *src = vec_at<const f32x4, const float>(p.bufs.p[r], a0);
#pragma unroll
                    for (int j = 0; j < VPT; ++j)
                        if (ok[j])
                            x[kk][j] = ld(src + vi[j]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                if (NT > 0 || k + kk < N) {
#pragma unroll
                    for (int j = 0; j < VPT; ++j)
                        if (ok[j])
                            acc[j] = acc[j] + x[kk][j];
                }
            }
        }
        const float fN = (float)N;
        f32x4 m[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            m[j] = acc[j] / fN;
        for (int n = 0; n < N; ++n) {
            f32x4 *dst = vec_at<f32x4, float>(p.bufs.p[n], a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                if (ok[j])
                    st(dst + vi[j], m[j]);
        }
        if (SGD) {
            f32x4 *wp = vec_at<f32x4, float>(p.w, a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                if (ok[j]) {
                    f32x4 wv = ld(wp + vi[j]);
                    const f32x4 step = p.lr * m[j];
                    wv = wv - step;
                    st(wp + vi[j], wv);
                }
            }
        }
    };

    run_span<4, VPT>(p.ct.off[c], p.ct.off[c + 1], elem, tile);
}

// ---------------------------------------------------------------------------
// Fused single pass, bfloat16 storage with binary32 arithmetic.
// ---------------------------------------------------------------------------

template <int NT, bool SGD>
__global__ __launch_bounds__(kThreads) void rar_fused_bf16(FusedParams p)
{
    constexpr int VPT = 1;
    const int N = NT > 0 ? NT : p.N;
    const int c = blockIdx.y;
    constexpr int KB = NT > 0 ? (NT > 1 ? NT - 1 : 1) : 8;

    auto elem = [&](int64_t e) {
        float acc = bf16_one(static_cast<const uint16_t *>(p.bufs.p[c])[e]);
        int r = c;
        for (int k = 1; k < N; ++k) {
            r = next_rank(r, N);
            acc = acc + bf16_one(static_cast<const uint16_t *>(p.bufs.p[r])[e]);
        }
        const float m = acc / (float)N;
        const uint16_t h = (uint16_t)bf16_rne(m);
        for (int n = 0; n < N; ++n)
            static_cast<uint16_t *>(p.bufs.p[n])[e] = h;
        if (SGD) {
            const float step = p.lr * m;
            p.w[e] = p.w[e] - step;
        }
    };

    auto tile = [&](auto full, int64_t a0, int64_t v0, int64_t nvec) {
        constexpr bool FULL = decltype(full)::value;
        int64_t vi[VPT];
        bool ok[VPT];
        lane_vectors<VPT, FULL>(v0, nvec, vi, ok);
        f32x4 lo[VPT], hi[VPT];
        {
            const u32x4 *src = vec_at<const u32x4, const uint16_t>(p.bufs.p[c], a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                if (ok[j])
                    widen8(ld(src + vi[j]), lo[j], hi[j]);
        }
        int r = c;
        for (int k = 1; k < N; k += KB) {
            u32x4 x[KB][VPT];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                if (NT > 0 || k + kk < N) {
                    r = next_rank(r, N);
                    const u32x4 *src = vec_at<const u32x4, const uint16_t>(p.bufs.p[r], a0);
#pragma unroll
                    for (int j = 0; j < VPT; ++j)
                        if (ok[j])
                            x[kk][j] = ld(src + vi[j]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                if (NT > 0 || k + kk < N) {
#pragma unroll
                    for (int j = 0; j < VPT; ++j) {
                        if (ok[j]) {
                            f32x4 a, b;
                            widen8(x[kk][j], a, b);
                            lo[j] = lo[j] + a;
                            hi[j] = hi[j] + b;
                        }
                    }
                }
            }
        }
        const float fN = (float)N;
        f32x4 mlo[VPT], mhi[VPT];
        u32x4 out[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            mlo[j] = lo[j] / fN;
            mhi[j] = hi[j] / fN;
            out[j] = narrow8(mlo[j], mhi[j]);
        }
        for (int n = 0; n < N; ++n) {
            u32x4 *dst = vec_at<u32x4, uint16_t>(p.bufs.p[n], a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                if (ok[j])
                    st(dst + vi[j], out[j]);
        }
        if (SGD) {
            f32x4 *wp = vec_at<f32x4, float>(p.w, a0);
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                if (ok[j]) {
                    f32x4 w0 = ld(wp + 2 * vi[j]);
                    f32x4 w1 = ld(wp + 2 * vi[j] + 1);
                    const f32x4 s0 = p.lr * mlo[j];
                    const f32x4 s1 = p.lr * mhi[j];
                    w0 = w0 - s0;
                    w1 = w1 - s1;
                    st(wp + 2 * vi[j], w0);
                    st(wp + 2 * vi[j] + 1, w1);
                }
            }
        }
    };

    run_span<8, VPT>(p.ct.off[c], p.ct.off[c + 1], elem, tile);
}

// ---------------------------------------------------------------------------
// Fused single pass with the work of one tile split over G lane groups.
// ---------------------------------------------------------------------------
//
// Same arithmetic as rar_fused_f32 / rar_fused_bf16, same bits.  A workgroup
// is G groups of kThreads lanes working on one tile of kThreads vectors.  The
// fold positions 0..N-1 of chunk c (rank (c+k) mod N at position k) are cut
// into G consecutive runs, one per group: every group loads only its run's
// vectors and, once the mean is known, stores only to its run's ranks; the
// last group also reads and writes w.  The partial sum passes from group to
// group through one LDS slot in fold order, so the additions happen in
// exactly the ring order; the last group divides by N and publishes the mean
// through a second slot.  G barriers per tile; LDS 8 KiB (binary32) or
// 16 KiB (bf16) whatever N is.
//
// Why: with one lane doing all N loads and N stores a lane has 2N+2 memory
// operations per tile.  Spreading them over G groups gives each wave fewer
// back-to-back stores, and HBM drains several concurrent write streams
// faster that way (measured on MI355X, 10 ranks x 300M with SGD: ~5.45 TB/s
// with one group, ~5.75 TB/s with two to four).
//
// How many memory operations a wave keeps in flight matters as well, and here
// it follows from how the group index is computed.  g = threadIdx.x / kThreads
// is not known to the compiler to be equal across a wave, so every lane loads
// its run's rank pointers from the kernel arguments itself, and the wait for
// each such pointer also waits for all of the wave's earlier loads and stores
// (one counter covers both): a wave's vector memory operations go out nearly
// one at a time.  On MI355X that is the fastest form measured.  A wave-uniform
// index (pointers in scalar registers, everything issued back to back) was
// 2.6% slower on 10 binary32 ranks and 3.7% slower on 40 bf16 ranks; explicit
// waits after each load or after each store, with the uniform index, came
// within 0.6% of this form on those two shapes, but lost up to 3.5% on bf16
// with two groups (8 and 16 ranks).  So g stays as it is.

// Scalar path for one element e of a span: the whole fold in one lane.
// base(r) is rank r's element pointer at the span's element 0.
template <typename T, int NT, bool SGD, class Base>
__device__ __forceinline__ void span_elem(Base base, float *w, float lr, int c, int64_t e)
{
    auto val = [&](int r) -> float {
        if constexpr (sizeof(T) == 4)
            return base(r)[e];
        else
            return bf16_one(base(r)[e]);
    };
    float acc = val(c);
    int r = c;
    for (int k = 1; k < NT; ++k) {
        r = next_rank(r, NT);
        acc = acc + val(r);
    }
    const float m = acc / (float)NT;
    for (int n = 0; n < NT; ++n) {
        if constexpr (sizeof(T) == 4)
            base(n)[e] = m;
        else
            base(n)[e] = (uint16_t)bf16_rne(m);
    }
    if (SGD) {
        const float step = lr * m;
        w[e] = w[e] - step;
    }
}

// Head and tail of a span: the elements before the first 128-byte aligned
// address of base(0) and after the last whole 16-byte group, on block
// bx == 0, lanes < 128/sizeof(T) (head) and the next VEC lanes (tail).
// Returns the head length h and the number of whole vectors nvec.
template <typename T, int NT, bool SGD, class Base>
__device__ __forceinline__ void span_head_tail(Base base, float *w, float lr, int c, int64_t len, int64_t bx,
                                               int64_t &h, int64_t &nvec)
{
    constexpr int VEC = 16 / sizeof(T);
    constexpr int LINE = 128 / sizeof(T);  // elements per 128-byte cache line
    const uintptr_t addr = reinterpret_cast<uintptr_t>(base(0));
    // The body starts on a cache line of rank 0, so each workgroup's tile
    // covers whole lines and no line is fetched by two workgroups (a chunk
    // of 2.5M bf16 elements starts 64 bytes into a line).  The other ranks
    // share rank 0's offset modulo 16 (modulo 128 for separate allocations).
    h = (int64_t)(((128 - (addr & 127)) & 127) / sizeof(T));
    if (h > len)
        h = len;
    nvec = (len - h) / VEC;
    const int64_t tail0 = h + nvec * VEC;
    if (bx != 0 || threadIdx.x >= LINE + VEC)
        return;
    const int64_t t = threadIdx.x;
    if (t < LINE) {
        if (t < h)
            span_elem<T, NT, SGD>(base, w, lr, c, t);
    } else if (t - LINE < len - tail0) {
        span_elem<T, NT, SGD>(base, w, lr, c, tail0 + (t - LINE));
    }
}

// The grouped body over one binary32 span of `len` elements whose fold starts
// at rank c; tiles bx, bx+gx, ... of the aligned part.
template <int NT, int G, bool SGD, class Base>
__device__ __forceinline__ void grouped_span_f32(Base base, float *w, float lr, int c, int64_t len, int64_t bx,
                                                 int64_t gx, f32x4 *chain, f32x4 *mean)
{
    static_assert(NT > 0 && G >= 1, "compile-time rank count");
    constexpr int PER = (NT + G - 1) / G;
    const int g = threadIdx.x / kThreads;
    const int lane = threadIdx.x % kThreads;
    const int k0 = g * PER;
    const int cnt = k0 >= NT ? 0 : (NT - k0 < PER ? NT - k0 : PER);
    int64_t h, nvec;
    span_head_tail<float, NT, SGD>(base, w, lr, c, len, bx, h, nvec);
    const int64_t ntiles = (nvec + kThreads - 1) / kThreads;
    for (int64_t t = bx; t < ntiles; t += gx) {
        const int64_t v = t * kThreads + lane;
        const bool ok = v < nvec;
        f32x4 x[PER];
        f32x4 wv = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (j < cnt) {
                    int r = c + k0 + j;
                    r = r >= NT ? r - NT : r;
                    x[j] = ld(reinterpret_cast<const f32x4 *>(base(r) + h) + v);
                }
            }
            if (SGD && g == G - 1)
                wv = ld(reinterpret_cast<const f32x4 *>(w + h) + v);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (g == 0 && ok) {
            acc = x[0];
#pragma unroll
            for (int j = 1; j < PER; ++j)
                if (j < cnt)
                    acc = acc + x[j];
        }
        f32x4 m;
        if constexpr (G > 1) {
#pragma unroll
            for (int hop = 1; hop < G; ++hop) {
                if (g == hop - 1)
                    chain[lane] = acc;
                __syncthreads();
                if (g == hop && ok) {
                    acc = chain[lane];
#pragma unroll
                    for (int j = 0; j < PER; ++j)
                        if (j < cnt)
                            acc = acc + x[j];
                }
            }
            if (g == G - 1)
                mean[lane] = acc / (float)NT;
            __syncthreads();
            m = mean[lane];
        } else {
            m = acc / (float)NT;
        }
        if (ok) {
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (j < cnt) {
                    int r = c + k0 + j;
                    r = r >= NT ? r - NT : r;
                    st(reinterpret_cast<f32x4 *>(base(r) + h) + v, m);
                }
            }
            if (SGD && g == G - 1) {
                const f32x4 step = lr * m;
                wv = wv - step;
                st(reinterpret_cast<f32x4 *>(w + h) + v, wv);
            }
        }
    }
}

// The same over a bf16 span (eight elements per 16-byte vector, binary32
// partial sums of 32 bytes per lane).
template <int NT, int G, bool SGD, class Base>
__device__ __forceinline__ void grouped_span_bf16(Base base, float *w, float lr, int c, int64_t len, int64_t bx,
                                                  int64_t gx, f32x4 *chain, f32x4 *mean)
{
    static_assert(NT > 0 && G >= 1, "compile-time rank count");
    constexpr int PER = (NT + G - 1) / G;
    const int g = threadIdx.x / kThreads;
    const int lane = threadIdx.x % kThreads;
    const int k0 = g * PER;
    const int cnt = k0 >= NT ? 0 : (NT - k0 < PER ? NT - k0 : PER);
    int64_t h, nvec;
    span_head_tail<uint16_t, NT, SGD>(base, w, lr, c, len, bx, h, nvec);
    const int64_t ntiles = (nvec + kThreads - 1) / kThreads;
    for (int64_t t = bx; t < ntiles; t += gx) {
        const int64_t v = t * kThreads + lane;
        const bool ok = v < nvec;
        u32x4 x[PER];
        f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (j < cnt) {
                    int r = c + k0 + j;
                    r = r >= NT ? r - NT : r;
                    x[j] = ld(reinterpret_cast<const u32x4 *>(base(r) + h) + v);
                }
            }
            if (SGD && g == G - 1) {
                const f32x4 *wp = reinterpret_cast<const f32x4 *>(w + h);
                w0 = ld(wp + 2 * v);
                w1 = ld(wp + 2 * v + 1);
            }
        }
        f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
        if (g == 0 && ok) {
            widen8(x[0], lo, hi);
#pragma unroll
            for (int j = 1; j < PER; ++j) {
                if (j < cnt) {
                    f32x4 a, b;
                    widen8(x[j], a, b);
                    lo = lo + a;
                    hi = hi + b;
                }
            }
        }
        f32x4 mlo, mhi;
        if constexpr (G > 1) {
#pragma unroll
            for (int hop = 1; hop < G; ++hop) {
                if (g == hop - 1) {
                    chain[2 * lane] = lo;
                    chain[2 * lane + 1] = hi;
                }
                __syncthreads();
                if (g == hop && ok) {
                    lo = chain[2 * lane];
                    hi = chain[2 * lane + 1];
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        if (j < cnt) {
                            f32x4 a, b;
                            // Emits nothing.  Without it the compiler widens each
                            // x[j] once for all G-1 unrolled hops and keeps the
                            // 2*PER binary32 vectors live instead of PER packed
                            // ones: past 128 VGPRs at N = 40, G = 4 (spills).
                            asm volatile("" : "+v"(x[j]));
                            widen8(x[j], a, b);
                            lo = lo + a;
                            hi = hi + b;
                        }
                    }
                }
            }
            if (g == G - 1) {
                mean[2 * lane] = lo / (float)NT;
                mean[2 * lane + 1] = hi / (float)NT;
            }
            __syncthreads();
            mlo = mean[2 * lane];
            mhi = mean[2 * lane + 1];
        } else {
            mlo = lo / (float)NT;
            mhi = hi / (float)NT;
        }
        if (ok) {
            const u32x4 out = narrow8(mlo, mhi);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                if (j < cnt) {
                    int r = c + k0 + j;
                    r = r >= NT ? r - NT : r;
                    st(reinterpret_cast<u32x4 *>(base(r) + h) + v, out);
                }
            }
            if (SGD && g == G - 1) {
                f32x4 *wp = reinterpret_cast<f32x4 *>(w + h);
                const f32x4 s0 = lr * mlo, s1 = lr * mhi;
                w0 = w0 - s0;
                w1 = w1 - s1;
                st(wp + 2 * v, w0);
                st(wp + 2 * v + 1, w1);
            }
        }
    }
}

// Flat rank buffers: span = chunk c = blockIdx.y of the chunk table.
template <int NT, int G, bool SGD>
__global__ __launch_bounds__(kThreads *G) void rar_fused_f32_grp(FusedParams p)
{
    __shared__ f32x4 chain[G > 1 ? kThreads : 1];
    __shared__ f32x4 mean[G > 1 ? kThreads : 1];
    const int c = blockIdx.y;
    const int64_t e0 = p.ct.off[c], e1 = p.ct.off[c + 1];
    if (e1 <= e0)
        return;
    auto base = [&](int r) { return static_cast<float *>(p.bufs.p[r]) + e0; };
    grouped_span_f32<NT, G, SGD>(base, SGD ? p.w + e0 : nullptr, p.lr, c, e1 - e0, blockIdx.x, gridDim.x, chain,
                                 mean);
}

template <int NT, int G, bool SGD>
__global__ __launch_bounds__(kThreads *G) void rar_fused_bf16_grp(FusedParams p)
{
    __shared__ f32x4 chain[G > 1 ? 2 * kThreads : 1];
    __shared__ f32x4 mean[G > 1 ? 2 * kThreads : 1];
    const int c = blockIdx.y;
    const int64_t e0 = p.ct.off[c], e1 = p.ct.off[c + 1];
    if (e1 <= e0)
        return;
    auto base = [&](int r) { return static_cast<uint16_t *>(p.bufs.p[r]) + e0; };
    grouped_span_bf16<NT, G, SGD>(base, SGD ? p.w + e0 : nullptr, p.lr, c, e1 - e0, blockIdx.x, gridDim.x, chain,
                                  mean);
}

// ---------------------------------------------------------------------------
// Buckets straight from the tensor lists.
// ---------------------------------------------------------------------------
//
// A bucket is a run of tensor segments cut into N chunks; a job is the part
// of one segment inside one chunk, so its fold starts at that chunk's rank
// and every rank's elements of the job are contiguous in that rank's tensor.
// Job j of rank r starts at ptr[j*N + r].  The same grouped body reduces each
// job in place in the tensors: no packing into bucket buffers and back, so a
// bucket moves 2*N*size bytes instead of 6*N*size.  vec_ok = 0 marks a job
// whose ranks' pointers differ in their 16-byte alignment; it goes through
// the scalar path.
template <typename T, int NT, int G>
__global__ __launch_bounds__(kThreads *G) void rar_bucket_jobs(JobsParams p)
{
    constexpr int SLOT = sizeof(T) == 4 ? 1 : 2;
    __shared__ f32x4 chain[G > 1 ? SLOT * kThreads : 1];
    __shared__ f32x4 mean[G > 1 ? SLOT * kThreads : 1];
    const int j = blockIdx.y;
    const JobDesc jd = p.job[j];
    auto base = [&](int r) { return static_cast<T *>(p.ptr[j * NT + r]); };
    if (jd.vec_ok) {
        if constexpr (sizeof(T) == 4)
            grouped_span_f32<NT, G, false>(base, nullptr, 0.f, jd.c, jd.len, blockIdx.x, gridDim.x, chain, mean);
        else
            grouped_span_bf16<NT, G, false>(base, nullptr, 0.f, jd.c, jd.len, blockIdx.x, gridDim.x, chain, mean);
    } else {
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < jd.len;
             e += (int64_t)gridDim.x * blockDim.x)
            span_elem<T, NT, false>(base, nullptr, 0.f, jd.c, e);
    }
}

// ---------------------------------------------------------------------------
// One scatter-reduce step, binary32, all N transfers of the step at once.
// ---------------------------------------------------------------------------
//
// [Gibiansky] §Scatter-reduce: at step s rank n sends chunk (n-s) mod N to
// rank n+1, which adds it into its own copy.  Seen from chunk c: the sender is
// rank (c+s) mod N and the receiver (c+s+1) mod N.  Within one step no rank
// reads and writes the same chunk, so the N transfers run concurrently in
// place.  The last step (s = N-2) completes the sum at the owner (c-1) mod N,
// which divides by N there and, with SGD, updates the weights of that chunk.

template <int VPT, bool LAST, bool SGD>
__global__ __launch_bounds__(kThreads) void rar_sr_step_f32(StepParams p)
{
    const int N = p.N;
    const int c = blockIdx.y;
    const int src = (c + p.s) % N;
    const int dst = (c + p.s + 1) % N;
    const float *sp = static_cast<const float *>(p.bufs.p[src]);
    float *dp = static_cast<float *>(p.bufs.p[dst]);
    float *w = p.sharded ? static_cast<float *>(p.wreps.p[dst]) : p.w;

    auto elem = [&](int64_t e) {
        float v = dp[e] + sp[e];
        if (LAST) {
            v = v / (float)N;
            if (SGD) {
                const float step = p.lr * v;
                w[e] = w[e] - step;
            }
        }
        dp[e] = v;
    };

    auto tile = [&](auto full, int64_t a0, int64_t v0, int64_t nvec) {
        constexpr bool FULL = decltype(full)::value;
        int64_t vi[VPT];
        bool ok[VPT];
        lane_vectors<VPT, FULL>(v0, nvec, vi, ok);
        const f32x4 *s4 = reinterpret_cast<const f32x4 *>(sp + a0);
        f32x4 *d4 = reinterpret_cast<f32x4 *>(dp + a0);
        f32x4 a[VPT], b[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (ok[j]) {
                a[j] = ld(d4 + vi[j]);
                b[j] = ld(s4 + vi[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (ok[j]) {
                f32x4 v = a[j] + b[j];
                if (LAST) {
                    v = v / (float)N;
                    if (SGD) {
                        f32x4 *w4 = reinterpret_cast<f32x4 *>(w + a0);
                        f32x4 wv = ld(w4 + vi[j]);
                        const f32x4 step = p.lr * v;
                        wv = wv - step;
                        st(w4 + vi[j], wv);
                    }
                }
                st(d4 + vi[j], v);
            }
        }
    };

    run_span<4, VPT>(p.ct.off[c], p.ct.off[c + 1], elem, tile);
}

// bf16 scatter-reduce step.  The running partial sum of chunk c travels in the
// binary32 workspace ws[C_c] (one holder per chunk at any step, so one
// chunk-indexed array serves all ranks).  FIRST: ws = own + sender's bf16;
// later: ws = own + ws; LAST: the owner's bf16 chunk receives the rounded
// mean, and the update uses the binary32 mean.
// Elements [e0, e1) of one transfer: sp, dp, ws (and w) are indexed by the
// same element index e.
template <bool FIRST, bool LAST, bool SGD>
__device__ __forceinline__ void sr_step_bf16_span(const uint16_t *sp, uint16_t *dp, float *ws, float *w, float lr,
                                                  int N, int64_t e0, int64_t e1)
{
    constexpr int VPT = 1;
    auto elem = [&](int64_t e) {
        const float incoming = FIRST ? bf16_one(sp[e]) : ws[e];
        const float v = bf16_one(dp[e]) + incoming;
        if (LAST) {
            const float m = v / (float)N;
            dp[e] = (uint16_t)bf16_rne(m);
            if (SGD) {
                const float step = lr * m;
                w[e] = w[e] - step;
            }
        } else {
            ws[e] = v;
        }
    };

    // The tile's 256 vectors (2048 elements) as 512 half-vectors of 4
    // elements: lane l takes half-vectors 2*v0 + l and 2*v0 + 256 + l.  Each
    // bf16 access is then 8 bytes and each binary32 access 16 bytes, both
    // contiguous across a wave, so no binary32 store instruction leaves
    // gaps (two interleaved 16-byte stores per lane measured 11% slower).
    auto tile = [&](auto full, int64_t a0, int64_t v0, int64_t nvec) {
        constexpr bool FULL = decltype(full)::value;
        const int64_t nh = 2 * nvec;
        const int64_t h[2] = {2 * v0 + threadIdx.x, 2 * v0 + kThreads + threadIdx.x};
        const bool ok[2] = {FULL || h[0] < nh, FULL || h[1] < nh};
        u32x2 *d8 = reinterpret_cast<u32x2 *>(dp + a0);
        const u32x2 *s8 = reinterpret_cast<const u32x2 *>(sp + a0);
        f32x4 *w4 = reinterpret_cast<f32x4 *>(ws + a0);
        f32x4 *wp = SGD ? reinterpret_cast<f32x4 *>(w + a0) : nullptr;
        f32x4 o[2], in[2], wv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!ok[k])
                continue;
            o[k] = widen4(ld(d8 + h[k]));
            in[k] = FIRST ? widen4(ld(s8 + h[k])) : ld(w4 + h[k]);
            if (LAST && SGD)
                wv[k] = ld(wp + h[k]);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!ok[k])
                continue;
            f32x4 sum = o[k] + in[k];
            if (LAST) {
                sum = sum / (float)N;
                st(d8 + h[k], narrow4(sum));
                if (SGD) {
                    const f32x4 step = lr * sum;
                    wv[k] = wv[k] - step;
                    st(wp + h[k], wv[k]);
                }
            } else {
                st(w4 + h[k], sum);
            }
        }
    };

    run_span<8, VPT>(e0, e1, elem, tile);
}

template <bool FIRST, bool LAST, bool SGD>
__global__ __launch_bounds__(kThreads) void rar_sr_step_bf16(StepParams p)
{
    const int N = p.N;
    const int c = blockIdx.y;
    const int src = (c + p.s) % N;
    const int dst = (c + p.s + 1) % N;
    sr_step_bf16_span<FIRST, LAST, SGD>(static_cast<const uint16_t *>(p.bufs.p[src]),
                                        static_cast<uint16_t *>(p.bufs.p[dst]), p.ws, p.w, p.lr, N, p.ct.off[c],
                                        p.ct.off[c + 1]);
}

// ---------------------------------------------------------------------------
// Scatter-reduce step over a table of pieces (buckets straight from the
// tensors): job j adds the sender's piece into the receiver's, elementwise;
// on the last step the receiver is the piece's owner and divides by N.  The
// pieces of one step are disjoint and none is both read and written in it
// ([Gibiansky] §Scatter-reduce, per chunk of each bucket), so one launch
// carries any number of them.
// ---------------------------------------------------------------------------

// One transfer of a ring step over n binary32 elements: ADD (scatter-reduce:
// the receiver's dp += the sender's sp, then / N when LAST) or a plain copy
// (all-gather: the receiver's dp = sp), tiles bx, bx+gx, ... of the body.
template <bool ADD, bool LAST>
__device__ __forceinline__ void step_span_f32(const float *sp, float *dp, int64_t n, float fN, int64_t bx,
                                              int64_t gx)
{
    auto elem = [&](int64_t e) {
        float v = ADD ? dp[e] + sp[e] : sp[e];
        if (LAST)
            v = v / fN;
        dp[e] = v;
    };
    if ((((uintptr_t)sp ^ (uintptr_t)dp) & 15) != 0) {
        // the two ranks' pieces differ in their 16-byte alignment
        for (int64_t e = bx * kThreads + threadIdx.x; e < n; e += gx * kThreads)
            elem(e);
        return;
    }
    // scalar elements up to the receiver's first 128-byte line (so no line is
    // written by two workgroups) and after the last whole 16-byte group
    int64_t h = (int64_t)(((128 - ((uintptr_t)dp & 127)) & 127) / 4);
    if (h > n)
        h = n;
    const int64_t nvec = (n - h) / 4;
    const int64_t tail0 = h + nvec * 4;
    if (bx == 0) {
        const int t = threadIdx.x;
        if (t < 32) {
            if (t < h)
                elem(t);
        } else if (t - 32 < n - tail0) {
            elem(tail0 + (t - 32));
        }
    }
    const f32x4 *s4 = reinterpret_cast<const f32x4 *>(sp + h);
    f32x4 *d4 = reinterpret_cast<f32x4 *>(dp + h);
    const int64_t ntiles = (nvec + kThreads - 1) / kThreads;
    for (int64_t t = bx; t < ntiles; t += gx) {
        const int64_t v = t * kThreads + threadIdx.x;
        if (v < nvec) {
            f32x4 x = ADD ? ld(d4 + v) + ld(s4 + v) : ld(s4 + v);
            if (LAST)
                x = x / fN;
            st(d4 + v, x);
        }
    }
}

template <bool LAST>
__global__ __launch_bounds__(kThreads) void rar_sr_jobs_f32(StepJobsParams p)
{
    const StepJob jb = p.job[blockIdx.y];
    step_span_f32<true, LAST>(jb.src, jb.dst, jb.len, (float)p.N, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// Consecutive buckets of per-rank arenas, one launch for all of them: row y
// of the grid is bucket y / N, chunk y % N, so no job table is needed.  The
// fused pass runs the grouped body of the flat kernels on each piece (fold
// from rank c, same bits); a ring step moves each piece from its sender to
// its receiver ([Gibiansky] §Scatter-reduce and §Allgather, per chunk of
// each bucket).
// ---------------------------------------------------------------------------

__device__ __forceinline__ void arena_piece(const ArenaParams &p, int k, int c, int64_t &e0, int64_t &len)
{
    const bool last = p.last_partial && k == p.nb - 1;
    const int64_t lo = last ? p.last.off[c] : p.full.off[c];
    const int64_t hi = last ? p.last.off[c + 1] : p.full.off[c + 1];
    e0 = (int64_t)k * p.B + lo;
    len = hi - lo;
}

template <typename T, int NT, int G>
__global__ __launch_bounds__(kThreads *G) void rar_arena_fused(ArenaParams p)
{
    constexpr int SLOT = sizeof(T) == 4 ? 1 : 2;
    __shared__ f32x4 chain[G > 1 ? SLOT * kThreads : 1];
    __shared__ f32x4 mean[G > 1 ? SLOT * kThreads : 1];
    const int k = blockIdx.y / NT, c = blockIdx.y % NT;
    int64_t e0, len;
    arena_piece(p, k, c, e0, len);
    if (len <= 0)
        return;
    auto base = [&](int r) { return static_cast<T *>(p.base[r]) + e0; };
    if constexpr (sizeof(T) == 4)
        grouped_span_f32<NT, G, false>(base, nullptr, 0.f, c, len, blockIdx.x, gridDim.x, chain, mean);
    else
        grouped_span_bf16<NT, G, false>(base, nullptr, 0.f, c, len, blockIdx.x, gridDim.x, chain, mean);
}

template <int OP>
__global__ __launch_bounds__(kThreads) void rar_arena_ring_f32(ArenaParams p)
{
    const int N = p.N;
    const int k = blockIdx.y / N, c = blockIdx.y - k * N;
    int64_t e0, len;
    arena_piece(p, k, c, e0, len);
    if (len <= 0)
        return;
    // scatter-reduce step s: rank (c+s) sends chunk c to rank (c+s+1);
    // all-gather step s: rank (c+s-1) sends it to rank (c+s)
    const int src = OP == kArenaAllgather ? (c + p.s - 1 + N) % N : (c + p.s) % N;
    const int dst = OP == kArenaAllgather ? (c + p.s) % N : (c + p.s + 1) % N;
    step_span_f32<OP != kArenaAllgather, OP == kArenaScatterReduceLast>(
        static_cast<const float *>(p.base[src]) + e0, static_cast<float *>(p.base[dst]) + e0, len, (float)N,
        blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// Multi-job copy: all-gather steps ([Gibiansky] §Allgather: the receiver
// overwrites), bucket pack/unpack, and the single reducer's broadcast.
// ---------------------------------------------------------------------------

// n bytes from s to d in units of `unit` (2 or 4) bytes; tiles bx, bx+gx, ...
template <int VPT>
__device__ __forceinline__ void copy_span(const char *s, char *d, int64_t n, int unit, int64_t bx, int64_t gx)
{
    auto copy_unit = [&](int64_t byte) {
        if (unit == 4)
            *reinterpret_cast<uint32_t *>(d + byte) = *reinterpret_cast<const uint32_t *>(s + byte);
        else
            *reinterpret_cast<uint16_t *>(d + byte) = *reinterpret_cast<const uint16_t *>(s + byte);
    };
    if (n <= 0)
        return;
    if ((((uintptr_t)s ^ (uintptr_t)d) & 15) == 0) {
        // same offset within a 16-byte group: scalar units up to the first
        // 128-byte line of d (so no line of d is written by two workgroups),
        // dwordx4 body, scalar units after the last 16-byte group
        const int64_t to_line = (int64_t)((128 - ((uintptr_t)d & 127)) & 127);
        const int64_t head = to_line < n ? to_line : n;
        const int64_t body = (n - head) / 16;
        const int64_t tail0 = head + body * 16;
        if (bx == 0) {
            const int64_t t = threadIdx.x;  // lanes 0..63: head units; 64..71: tail units
            if (t < 64) {
                if (t * unit < head)
                    copy_unit(t * unit);
            } else if (t < 72 && (t - 64) * unit < n - tail0) {
                copy_unit(tail0 + (t - 64) * unit);
            }
        }
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(s + head);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(d + head);
        constexpr int64_t TV = (int64_t)kThreads * VPT;
        const int64_t ntiles = (body + TV - 1) / TV;
        for (int64_t t = bx; t < ntiles; t += gx) {
            const int64_t v0 = t * TV;
            u32x4 x[VPT];
            if (v0 + TV <= body) {
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    x[j] = ld(s4 + v0 + (int64_t)j * kThreads + threadIdx.x);
#pragma unroll
                for (int j = 0; j < VPT; ++j)
                    st(d4 + v0 + (int64_t)j * kThreads + threadIdx.x, x[j]);
            } else {
#pragma unroll
                for (int j = 0; j < VPT; ++j) {
                    const int64_t v = v0 + (int64_t)j * kThreads + threadIdx.x;
                    if (v < body)
                        st(d4 + v, ld(s4 + v));
                }
            }
        }
    } else {
        const int64_t units = n / unit;
        for (int64_t i = bx * kThreads + threadIdx.x; i < units; i += gx * kThreads)
            copy_unit(i * unit);
    }
}

template <int VPT>
__global__ __launch_bounds__(kThreads) void rar_copy(CopyParams p)
{
    const CopyJob job = p.job[blockIdx.y];
    copy_span<VPT>(static_cast<const char *>(job.src), static_cast<char *>(job.dst), job.nbytes, p.unit, blockIdx.x,
                   gridDim.x);
}

// A ring step over every chunk of every bucket of bf16 arenas: the
// scatter-reduce carries each chunk's binary32 partial sum in ws (one holder
// per chunk at any step, so one array indexed like the arenas serves every
// rank), the last step writes the owner's rounded mean, and the all-gather
// copies it on ([Gibiansky] §Scatter-reduce and §Allgather, per chunk of each
// bucket).
template <int OP>
__global__ __launch_bounds__(kThreads) void rar_arena_ring_bf16(ArenaParams p)
{
    const int N = p.N;
    const int k = blockIdx.y / N, c = blockIdx.y - k * N;
    int64_t e0, len;
    arena_piece(p, k, c, e0, len);
    if (len <= 0)
        return;
    const int src = OP == kArenaAllgather ? (c + p.s - 1 + N) % N : (c + p.s) % N;
    const int dst = OP == kArenaAllgather ? (c + p.s) % N : (c + p.s + 1) % N;
    const uint16_t *sp = static_cast<const uint16_t *>(p.base[src]);
    uint16_t *dp = static_cast<uint16_t *>(p.base[dst]);
    if constexpr (OP == kArenaAllgather) {
        copy_span<1>(reinterpret_cast<const char *>(sp + e0), reinterpret_cast<char *>(dp + e0), len * 2, 2,
                     blockIdx.x, gridDim.x);
    } else {
        constexpr bool FIRST = OP == kArenaScatterReduceFirst || OP == kArenaScatterReduceFirstLast;
        constexpr bool LAST = OP == kArenaScatterReduceLast || OP == kArenaScatterReduceFirstLast;
        sr_step_bf16_span<FIRST, LAST, false>(sp, dp, p.ws, nullptr, 0.f, N, e0, e0 + len);
    }
}

// ---------------------------------------------------------------------------
// Single reducer (prior art): rank 0 adds rank `src`; the last addition also
// divides by N and applies SGD.  Summation order g0 + g1 + ... + g(N-1).
// ---------------------------------------------------------------------------

template <int VPT, bool LAST, bool SGD>
__global__ __launch_bounds__(kThreads) void rar_reduce_into_rank0_f32(PairParams p)
{
    const int N = p.N;
    const float *sp = static_cast<const float *>(p.bufs.p[p.src]);
    float *dp = static_cast<float *>(p.bufs.p[0]);
    float *w = p.w;
    auto elem = [&](int64_t e) {
        float v = dp[e] + sp[e];
        if (LAST) {
            v = v / (float)N;
            if (SGD) {
                const float step = p.lr * v;
                w[e] = w[e] - step;
            }
        }
        dp[e] = v;
    };
    auto tile = [&](auto full, int64_t a0, int64_t v0, int64_t nvec) {
        constexpr bool FULL = decltype(full)::value;
        int64_t vi[VPT];
        bool ok[VPT];
        lane_vectors<VPT, FULL>(v0, nvec, vi, ok);
        const f32x4 *s4 = reinterpret_cast<const f32x4 *>(sp + a0);
        f32x4 *d4 = reinterpret_cast<f32x4 *>(dp + a0);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (ok[j]) {
                f32x4 v = ld(d4 + vi[j]) + ld(s4 + vi[j]);
                if (LAST) {
                    v = v / (float)N;
                    if (SGD) {
                        f32x4 *w4 = reinterpret_cast<f32x4 *>(w + a0);
                        f32x4 wv = ld(w4 + vi[j]);
                        const f32x4 step = p.lr * v;
                        wv = wv - step;
                        st(w4 + vi[j], wv);
                    }
                }
                st(d4 + vi[j], v);
            }
        }
    };
    run_span<4, VPT>(0, p.P, elem, tile);
}

// ---------------------------------------------------------------------------
// Launch shapes
// ---------------------------------------------------------------------------

// Blocks along x for `jobs` jobs of at most `max_vecs` 16-byte vectors each:
// by default one tile per workgroup (measured on MI355X: a launch of one tile
// per workgroup streams ~11% faster than a grid-stride loop over 8
// workgroups per CU, because more independent waves keep more requests in
// flight); a plan may cap the total, which turns on the grid-stride loop.
int blocks_x(int max_blocks, int jobs, int64_t max_vecs, int vpt)
{
    const int64_t per_tile = (int64_t)kThreads * vpt;
    int64_t need = (max_vecs + per_tile - 1) / per_tile;
    if (need < 1)
        need = 1;
    int64_t bx = ((int64_t)max_blocks + jobs - 1) / jobs;
    if (bx < 1)
        bx = 1;
    if (bx > need)
        bx = need;
    // x may exceed 65535 (only y, the job, may not); a dispatch counts its
    // work-items in 32 bits, so x times up to 1024 lanes stays below 2^32
    if (bx > (1 << 22) - 1)
        bx = (1 << 22) - 1;
    return (int)bx;
}

// Lane groups per workgroup of the grouped fused kernels, by rank count and
// element type, from a sweep on MI355X over 1-4 groups (fused pass with and
// without SGD at 4, 8, 10, 16 and 40 ranks): binary32 gains from splitting a
// tile over up to four groups; bf16, with twice the elements and the widening
// per lane and a 32-byte partial sum to pass, gains from two groups at
// 4-16 ranks and from four at 40 (where two are far slower, and four fit in
// the registers only with the empty asm in its hop loop).
constexpr int groups_f32(int N) { return N <= 3 ? 1 : N <= 4 ? 2 : N <= 12 ? 4 : N <= 16 ? 3 : 4; }
constexpr int groups_bf16(int N) { return N <= 3 ? 1 : N <= 16 ? 2 : 4; }

template <int NT>
hipError_t fused_grouped(rar_dtype dt, const FusedParams &p, int max_blocks, int64_t max_chunk,
                         hipStream_t st)
{
    const bool sgd = p.w != nullptr;
    if (dt == RAR_F32) {
        constexpr int G = groups_f32(NT);
        const dim3 g(blocks_x(max_blocks, NT, max_chunk / 4 + 1, 1), NT), b(kThreads * G);
        if (sgd)
            hipLaunchKernelGGL((rar_fused_f32_grp<NT, G, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_fused_f32_grp<NT, G, false>), g, b, 0, st, p);
    } else {
        constexpr int G = groups_bf16(NT);
        const dim3 g(blocks_x(max_blocks, NT, max_chunk / 8 + 1, 1), NT), b(kThreads * G);
        if (sgd)
            hipLaunchKernelGGL((rar_fused_bf16_grp<NT, G, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_fused_bf16_grp<NT, G, false>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

template <int NT>
hipError_t bucket_jobs_n(rar_dtype dt, const JobsParams &p, int max_blocks, int64_t max_len, hipStream_t st)
{
    if (dt == RAR_F32) {
        constexpr int G = groups_f32(NT);
        const dim3 g(blocks_x(max_blocks, p.njobs, max_len / 4 + 1, 1), p.njobs), b(kThreads * G);
        hipLaunchKernelGGL((rar_bucket_jobs<float, NT, G>), g, b, 0, st, p);
    } else {
        constexpr int G = groups_bf16(NT);
        const dim3 g(blocks_x(max_blocks, p.njobs, max_len / 8 + 1, 1), p.njobs), b(kThreads * G);
        hipLaunchKernelGGL((rar_bucket_jobs<uint16_t, NT, G>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace

// The static workspace: binary32 partial sums of a bf16 ring for callers that
// cannot allocate.  In host code `scratch` names a host-side stand-in, not
// device memory; only the address hipGetSymbolAddress returns for the current
// device is ever handed to a kernel.
static __device__ __align__(256) float scratch[RAR_STATIC_WS_ELEMS];

hipError_t static_workspace(int device, float **ptr)
{
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[device] = static_cast<float *>(p);
    }
    *ptr = addr[device];
    return hipSuccess;
}

bool bucket_jobs_supported(int N)
{
    return N == 2 || N == 4 || N == 8 || N == 10 || N == 16 || N == 40;
}

hipError_t launch_bucket_jobs(rar_dtype dt, int N, const JobsParams &p, int max_blocks, int64_t max_len,
                              hipStream_t st)
{
    if (p.njobs <= 0)
        return hipSuccess;
    switch (N) {
    case 2: return bucket_jobs_n<2>(dt, p, max_blocks, max_len, st);
    case 4: return bucket_jobs_n<4>(dt, p, max_blocks, max_len, st);
    case 8: return bucket_jobs_n<8>(dt, p, max_blocks, max_len, st);
    case 10: return bucket_jobs_n<10>(dt, p, max_blocks, max_len, st);
    case 16: return bucket_jobs_n<16>(dt, p, max_blocks, max_len, st);
    case 40: return bucket_jobs_n<40>(dt, p, max_blocks, max_len, st);
    default: return hipErrorInvalidValue;
    }
}

// Rank counts with a compile-time kernel (the workloads' 4, 8, 10 and 40, and
// the powers of two up to 16) take the grouped kernels; any other N takes the
// runtime-N single-group kernels.
hipError_t launch_fused(rar_dtype dt, const FusedParams &p, int max_blocks, int64_t max_chunk,
                        hipStream_t st)
{
    switch (p.N) {
    case 2: return fused_grouped<2>(dt, p, max_blocks, max_chunk, st);
    case 4: return fused_grouped<4>(dt, p, max_blocks, max_chunk, st);
    case 8: return fused_grouped<8>(dt, p, max_blocks, max_chunk, st);
    case 10: return fused_grouped<10>(dt, p, max_blocks, max_chunk, st);
    case 16: return fused_grouped<16>(dt, p, max_blocks, max_chunk, st);
    case 40: return fused_grouped<40>(dt, p, max_blocks, max_chunk, st);
    default: break;
    }
    const bool sgd = p.w != nullptr;
    const dim3 b(kThreads);
    if (dt == RAR_F32) {
        const dim3 g(blocks_x(max_blocks, p.N, max_chunk / 4 + 1, 1), p.N);
        if (sgd)
            hipLaunchKernelGGL((rar_fused_f32<0, 1, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_fused_f32<0, 1, false>), g, b, 0, st, p);
    } else {
        const dim3 g(blocks_x(max_blocks, p.N, max_chunk / 8 + 1, 1), p.N);
        if (sgd)
            hipLaunchKernelGGL((rar_fused_bf16<0, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_fused_bf16<0, false>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_sr_step(rar_dtype dt, const StepParams &p, bool first, bool last, bool sgd,
                          int max_blocks, int64_t max_chunk, hipStream_t st)
{
    const dim3 b(kThreads);
    if (dt == RAR_F32) {
        constexpr int VPT = 1;
        const dim3 g(blocks_x(max_blocks, p.N, max_chunk / 4 + 1, VPT), p.N);
        if (!last)
            hipLaunchKernelGGL((rar_sr_step_f32<VPT, false, false>), g, b, 0, st, p);
        else if (sgd)
            hipLaunchKernelGGL((rar_sr_step_f32<VPT, true, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_sr_step_f32<VPT, true, false>), g, b, 0, st, p);
        return hipGetLastError();
    }
    const dim3 g(blocks_x(max_blocks, p.N, max_chunk / 8 + 1, 1), p.N);
    if (first && last) {
        if (sgd)
            hipLaunchKernelGGL((rar_sr_step_bf16<true, true, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_sr_step_bf16<true, true, false>), g, b, 0, st, p);
    } else if (first) {
        hipLaunchKernelGGL((rar_sr_step_bf16<true, false, false>), g, b, 0, st, p);
    } else if (last) {
        if (sgd)
            hipLaunchKernelGGL((rar_sr_step_bf16<false, true, true>), g, b, 0, st, p);
        else
            hipLaunchKernelGGL((rar_sr_step_bf16<false, true, false>), g, b, 0, st, p);
    } else {
        hipLaunchKernelGGL((rar_sr_step_bf16<false, false, false>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_sr_jobs(const StepJobsParams &p, bool last, int64_t max_len, hipStream_t st)
{
    if (p.njobs <= 0)
        return hipSuccess;
    const dim3 g(blocks_x(1 << 24, p.njobs, max_len / 4 + 1, 1), p.njobs);
    if (last)
        hipLaunchKernelGGL((rar_sr_jobs_f32<true>), g, dim3(kThreads), 0, st, p);
    else
        hipLaunchKernelGGL((rar_sr_jobs_f32<false>), g, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <int NT>
hipError_t arena_fused_n(rar_dtype dt, const ArenaParams &p, int64_t max_chunk, hipStream_t st)
{
    const int rows = p.nb * NT;
    if (dt == RAR_F32) {
        constexpr int G = groups_f32(NT);
        const dim3 g(blocks_x(1 << 24, rows, max_chunk / 4 + 1, 1), rows), b(kThreads * G);
        hipLaunchKernelGGL((rar_arena_fused<float, NT, G>), g, b, 0, st, p);
    } else {
        constexpr int G = groups_bf16(NT);
        const dim3 g(blocks_x(1 << 24, rows, max_chunk / 8 + 1, 1), rows), b(kThreads * G);
        hipLaunchKernelGGL((rar_arena_fused<uint16_t, NT, G>), g, b, 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_arena(rar_dtype dt, ArenaOp op, const ArenaParams &p, int64_t max_chunk, hipStream_t st)
{
    if (p.nb <= 0)
        return hipSuccess;
    if (op == kArenaFused) {
        switch (p.N) {
        case 2: return arena_fused_n<2>(dt, p, max_chunk, st);
        case 4: return arena_fused_n<4>(dt, p, max_chunk, st);
        case 8: return arena_fused_n<8>(dt, p, max_chunk, st);
        case 10: return arena_fused_n<10>(dt, p, max_chunk, st);
        case 16: return arena_fused_n<16>(dt, p, max_chunk, st);
        case 40: return arena_fused_n<40>(dt, p, max_chunk, st);
        default: return hipErrorInvalidValue;
        }
    }
    if (p.N < 2)
        return hipErrorInvalidValue;
    const int rows = p.nb * p.N;
    if (dt == RAR_BF16) {
        if (!p.ws)
            return hipErrorInvalidValue;
        const dim3 g(blocks_x(1 << 24, rows, max_chunk / 8 + 1, 1), rows), b(kThreads);
        switch (op) {
        case kArenaScatterReduceFirst: hipLaunchKernelGGL((rar_arena_ring_bf16<kArenaScatterReduceFirst>), g, b, 0, st, p); break;
        case kArenaScatterReduceFirstLast:
            hipLaunchKernelGGL((rar_arena_ring_bf16<kArenaScatterReduceFirstLast>), g, b, 0, st, p);
            break;
        case kArenaScatterReduce: hipLaunchKernelGGL((rar_arena_ring_bf16<kArenaScatterReduce>), g, b, 0, st, p); break;
        case kArenaScatterReduceLast: hipLaunchKernelGGL((rar_arena_ring_bf16<kArenaScatterReduceLast>), g, b, 0, st, p); break;
        case kArenaAllgather: hipLaunchKernelGGL((rar_arena_ring_bf16<kArenaAllgather>), g, b, 0, st, p); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    // binary32 partial sums live in the arenas themselves: the first step is a middle one
    if (op == kArenaScatterReduceFirst)
        op = kArenaScatterReduce;
    else if (op == kArenaScatterReduceFirstLast)
        op = kArenaScatterReduceLast;
    const dim3 g(blocks_x(1 << 24, rows, max_chunk / 4 + 1, 1), rows);
    switch (op) {
    case kArenaScatterReduce: hipLaunchKernelGGL((rar_arena_ring_f32<kArenaScatterReduce>), g, dim3(kThreads), 0, st, p); break;
    case kArenaScatterReduceLast:
        hipLaunchKernelGGL((rar_arena_ring_f32<kArenaScatterReduceLast>), g, dim3(kThreads), 0, st, p);
        break;
    default: hipLaunchKernelGGL((rar_arena_ring_f32<kArenaAllgather>), g, dim3(kThreads), 0, st, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_copy(const CopyParams &p, int max_blocks, int64_t max_job_bytes, hipStream_t st)
{
    if (p.njobs <= 0)
        return hipSuccess;
    constexpr int VPT = 1;
    const dim3 g(blocks_x(max_blocks, p.njobs, max_job_bytes / 16 + 1, VPT), p.njobs);
    hipLaunchKernelGGL((rar_copy<VPT>), g, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_pair_add(const PairParams &p, bool last, bool sgd, int max_blocks, hipStream_t st)
{
    constexpr int VPT = 1;
    const dim3 g(blocks_x(max_blocks, 1, p.P / 4 + 1, VPT), 1);
    const dim3 b(kThreads);
    if (!last)
        hipLaunchKernelGGL((rar_reduce_into_rank0_f32<VPT, false, false>), g, b, 0, st, p);
    else if (sgd)
        hipLaunchKernelGGL((rar_reduce_into_rank0_f32<VPT, true, true>), g, b, 0, st, p);
    else
        hipLaunchKernelGGL((rar_reduce_into_rank0_f32<VPT, true, false>), g, b, 0, st, p);
    return hipGetLastError();
}

}  // namespace rar
