"""Python binding of librar.so: one function per C entry point, same names.

Argument marshalling only -- every step of the all-reduce runs in the HIP
library.  Device buffers may be given as torch tensors (contiguous, on the
GPU, of the plan's element type: float32 for RAR_F32 and for weights,
bfloat16 for RAR_BF16, with at least as many elements as the call touches;
ValueError otherwise) or as integer device addresses, which are passed on
unchecked.  ``stream`` may be a torch stream, an
integer hipStream_t, or None for torch's current stream on the current
device (the default stream when torch has no GPU).

Status codes other than RAR_OK raise RarError carrying the code.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

from ._lib import lib

# enums of rar.h
F32, BF16 = 0, 1
BALANCED, CEIL, ALIGN16 = 0, 1, 2
FUSED, RING, NAIVE = 0, 1, 2
OK, EINVAL, EMISMATCH, EALIGN, ENOMEM, EHIP, ETOOLARGE = 0, -1, -2, -3, -4, -5, -6
MAX_RANKS = 64
MAX_STRIDE_CANDIDATES = 64
STATIC_WS_ELEMS = 1 << 24


class RarError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {rar_strerror(status)} ({status})")


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise RarError(rc, where)


def rar_strerror(status: int) -> str:
    return lib().rar_strerror(int(status)).decode()


def rar_version() -> int:
    return int(lib().rar_version())


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("tensor must be contiguous")
        if x.numel() and not x.is_cuda:
            raise ValueError("tensor must be on the GPU")
        return int(x.data_ptr())
    raise TypeError(f"not a device buffer: {type(x)!r}")


def _ptr_array(xs: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(len(xs), 1))()
    for i, x in enumerate(xs):
        arr[i] = _addr(x) or None
    return arr


def _ranks(xs: Sequence, N: int, what: str) -> ctypes.Array:
    # the library reads exactly N pointers from the array
    if len(xs) != N:
        raise ValueError(f"{what}: {len(xs)} entries for {N} ranks")
    return _ptr_array(xs)


_DTYPES = {}


def _torch_dtype(dtype: int):
    if dtype not in _DTYPES:
        import torch
        _DTYPES[dtype] = torch.float32 if dtype == F32 else torch.bfloat16
    return _DTYPES[dtype]


def _check_tensor(x, what: str, dtype: int, min_numel: int) -> None:
    """A tensor argument must have the element type the library will read and
    write through it, and at least as many elements as it will touch (the
    library sees only an address).  Integer addresses are taken as given."""
    if x is None or isinstance(x, int) or not hasattr(x, "data_ptr"):
        return
    want = _torch_dtype(dtype)
    if x.dtype != want:
        raise ValueError(f"{what}: dtype {x.dtype}, expected {want}")
    if x.numel() < min_numel:
        raise ValueError(f"{what}: {x.numel()} elements, at least {min_numel} needed")


def _check_ranks(xs: Sequence, what: str, dtype: int, min_numel: int) -> None:
    for n, x in enumerate(xs):
        if hasattr(x, "data_ptr") and (x.dtype != _torch_dtype(dtype) or x.numel() < min_numel):
            _check_tensor(x, f"{what}[{n}]", dtype, min_numel)  # raises, with the argument's name


def _stream(s) -> int:
    if s is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except ImportError:
            pass
        return 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"not a stream: {type(s)!r}")


# ---------------------------------------------------------------------------
# Plans
# ---------------------------------------------------------------------------

class Plan:
    """Owner of a rar_plan_t; destroyed with the object or by rar_plan_destroy."""

    def __init__(self, handle: int, N: int, P: int, dtype: int, chunking: int):
        self.handle = ctypes.c_void_p(handle)
        self.N, self.P, self.dtype, self.chunking = N, P, dtype, chunking

    def __del__(self):
        try:
            rar_plan_destroy(self)
        except Exception:
            pass


def rar_plan(N: int, P: int, dtype: int = F32, chunking: int = BALANCED) -> Plan:
    out = ctypes.c_void_p()
    _check(lib().rar_plan(int(N), int(P), int(dtype), int(chunking), ctypes.byref(out)), "rar_plan")
    return Plan(out.value, int(N), int(P), int(dtype), int(chunking))


def rar_rank_stride(P: int, dtype: int = F32) -> int:
    """Recommended byte distance between rank buffers carved from one allocation."""
    out = ctypes.c_int64()
    _check(lib().rar_rank_stride(int(P), int(dtype), ctypes.byref(out)), "rar_rank_stride")
    return out.value


def rar_rank_stride_candidate(P: int, dtype: int, k: int) -> int:
    """Candidate k of the strides rar_rank_stride_tune times (for sizing its pool)."""
    out = ctypes.c_int64()
    _check(lib().rar_rank_stride_candidate(int(P), int(dtype), int(k), ctypes.byref(out)),
           "rar_rank_stride_candidate")
    return out.value


def rar_rank_stride_tune(N: int, P: int, dtype: int, pool, candidates: int = 64, stream=None) -> int:
    """Measured byte distance between rank buffers carved from `pool` (a
    device tensor or pointer; its contents are overwritten).  Waits for the
    stream."""
    out = ctypes.c_int64()
    nbytes = pool.numel() * pool.element_size() if hasattr(pool, "element_size") else None
    if nbytes is None:
        raise TypeError("pool must be a tensor (its size bounds the candidates)")
    _check(lib().rar_rank_stride_tune(int(N), int(P), int(dtype), _addr(pool), int(nbytes), int(candidates),
                                      _stream(stream), ctypes.byref(out)), "rar_rank_stride_tune")
    return out.value


def rar_rank_stride_tune_stats(N: int, P: int, dtype: int, pool, candidates: int = 64, stream=None):
    """rar_rank_stride_tune and its measurements: (stride, [(candidate stride,
    median ms, spread ms), ...])."""
    if not hasattr(pool, "element_size"):
        raise TypeError("pool must be a tensor (its size bounds the candidates)")
    nbytes = pool.numel() * pool.element_size()
    out, K = ctypes.c_int64(), ctypes.c_int()
    cs = (ctypes.c_int64 * candidates)()
    med, spr = (ctypes.c_float * candidates)(), (ctypes.c_float * candidates)()
    _check(lib().rar_rank_stride_tune_stats(int(N), int(P), int(dtype), _addr(pool), int(nbytes), int(candidates),
                                            _stream(stream), ctypes.byref(out), ctypes.byref(K), cs, med, spr),
           "rar_rank_stride_tune_stats")
    return out.value, [(cs[k], med[k], spr[k]) for k in range(K.value)]


def rar_plan_destroy(plan: Plan) -> None:
    if plan.handle:
        h, plan.handle = plan.handle, ctypes.c_void_p()
        _check(lib().rar_plan_destroy(h), "rar_plan_destroy")


def rar_plan_set_algo(plan: Plan, algo: int) -> None:
    _check(lib().rar_plan_set_algo(plan.handle, int(algo)), "rar_plan_set_algo")


def rar_plan_set_grid(plan: Plan, max_blocks: int) -> None:
    _check(lib().rar_plan_set_grid(plan.handle, int(max_blocks)), "rar_plan_set_grid")


def rar_plan_chunk(plan: Plan, c: int):
    off, ln, own = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    _check(lib().rar_plan_chunk(plan.handle, int(c), ctypes.byref(off), ctypes.byref(ln), ctypes.byref(own)),
           "rar_plan_chunk")
    return off.value, ln.value, own.value


def rar_plan_traffic(plan: Plan, rank: int):
    s, r = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().rar_plan_traffic(plan.handle, int(rank), ctypes.byref(s), ctypes.byref(r)), "rar_plan_traffic")
    return s.value, r.value


# ---------------------------------------------------------------------------
# All-reduce
# ---------------------------------------------------------------------------

def _check_exec(plan: Plan, bufs: Sequence, P: int) -> None:
    # a P that differs from the plan's is the library's RAR_EMISMATCH, raised
    # before it touches any buffer
    if int(P) == plan.P:
        _check_ranks(bufs, "bufs", plan.dtype, plan.P)


def _check_weights(w, what: str, plan: Plan, P: int) -> None:
    if int(P) == plan.P:
        _check_tensor(w, what, F32, plan.P)


def rar_allreduce_mean(plan: Plan, bufs: Sequence, P: int, stream=None) -> None:
    _check_exec(plan, bufs, P)
    _check(lib().rar_allreduce_mean(plan.handle, _ranks(bufs, plan.N, "bufs"), int(P), _stream(stream)),
           "rar_allreduce_mean")


def rar_allreduce_sgd(plan: Plan, bufs: Sequence, w, lr: float, P: int, stream=None) -> None:
    _check_exec(plan, bufs, P)
    _check_weights(w, "w", plan, P)
    _check(lib().rar_allreduce_sgd(plan.handle, _ranks(bufs, plan.N, "bufs"), _addr(w), ctypes.c_float(lr), int(P),
                                   _stream(stream)), "rar_allreduce_sgd")


def rar_allreduce_ring_noalloc(plan: Plan, bufs: Sequence, w, lr: float, P: int, stream=None) -> None:
    """The ring all-reduce-mean (w None) or + SGD with no device allocation:
    a bf16 plan's partial sums use the library's static workspace."""
    _check_exec(plan, bufs, P)
    if w is not None:
        _check_weights(w, "w", plan, P)
    _check(lib().rar_allreduce_ring_noalloc(plan.handle, _ranks(bufs, plan.N, "bufs"), _addr(w),
                                            ctypes.c_float(lr), int(P), _stream(stream)),
           "rar_allreduce_ring_noalloc")


def rar_reduce_scatter_sgd_allgather(plan: Plan, bufs: Sequence, w_reps: Sequence, lr: float, P: int,
                                     stream=None) -> None:
    _check_exec(plan, bufs, P)
    for n, w in enumerate(w_reps):
        _check_weights(w, f"w_reps[{n}]", plan, P)
    _check(lib().rar_reduce_scatter_sgd_allgather(plan.handle, _ranks(bufs, plan.N, "bufs"),
                                                  _ranks(w_reps, plan.N, "w_reps"),
                                                  ctypes.c_float(lr), int(P), _stream(stream)),
           "rar_reduce_scatter_sgd_allgather")


# ---------------------------------------------------------------------------
# Buckets
# ---------------------------------------------------------------------------

class Buckets:
    def __init__(self, handle: int, numel: Sequence[int], dtype: int):
        self.handle = ctypes.c_void_p(handle)
        self.numel = [int(n) for n in numel]
        self.n_tensors, self.dtype, self.total = len(self.numel), dtype, sum(self.numel)

    def __del__(self):
        try:
            rar_bucket_destroy(self)
        except Exception:
            pass


def rar_bucket_plan(numel: Sequence[int], dtype: int = F32, bucket_bytes: int = 25_000_000) -> Buckets:
    arr = (ctypes.c_int64 * max(len(numel), 1))(*[int(n) for n in numel])
    out = ctypes.c_void_p()
    _check(lib().rar_bucket_plan(len(numel), arr, int(dtype), int(bucket_bytes), ctypes.byref(out)),
           "rar_bucket_plan")
    return Buckets(out.value, numel, int(dtype))


def rar_bucket_destroy(b: Buckets) -> None:
    if b.handle:
        h, b.handle = b.handle, ctypes.c_void_p()
        _check(lib().rar_bucket_destroy(h), "rar_bucket_destroy")


def rar_bucket_count(b: Buckets):
    n, m = ctypes.c_int(), ctypes.c_int64()
    _check(lib().rar_bucket_count(b.handle, ctypes.byref(n), ctypes.byref(m)), "rar_bucket_count")
    return n.value, m.value


def rar_bucket_info(b: Buckets, bucket: int):
    so, el, ns = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    _check(lib().rar_bucket_info(b.handle, int(bucket), ctypes.byref(so), ctypes.byref(el), ctypes.byref(ns)),
           "rar_bucket_info")
    return so.value, el.value, ns.value


def rar_bucket_segment(b: Buckets, bucket: int, seg: int):
    t, to, bo, ln = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().rar_bucket_segment(b.handle, int(bucket), int(seg), ctypes.byref(t), ctypes.byref(to),
                                    ctypes.byref(bo), ctypes.byref(ln)), "rar_bucket_segment")
    return t.value, to.value, bo.value, ln.value


def _rank_major(b: "Buckets", tensors: Sequence[Sequence]) -> ctypes.Array:
    # the library reads N * n_tensors pointers: every rank must list them all
    want, numel = _torch_dtype(b.dtype), b.numel
    for n, rank in enumerate(tensors):
        if len(rank) != b.n_tensors:
            raise ValueError(f"rank {n} lists {len(rank)} tensors; the bucket plan has {b.n_tensors}")
        for t, x in enumerate(rank):
            # the common case costs two comparisons; the message is built only on failure
            if hasattr(x, "data_ptr") and (x.dtype != want or x.numel() < numel[t]):
                _check_tensor(x, f"tensors[{n}][{t}]", b.dtype, numel[t])
    flat = [x for rank in tensors for x in rank]
    return _ptr_array(flat)


def _check_bucket_bufs(b: Buckets, bucket_bufs: Sequence, elems: int) -> None:
    _check_ranks(bucket_bufs, "bucket_bufs", b.dtype, elems)


def _bucket_elems(b: Buckets, bucket: int) -> int:
    # a bad bucket index is the library's RAR_EINVAL
    nb = rar_bucket_count(b)[0] if b.handle else 0
    return rar_bucket_info(b, bucket)[1] if 0 <= int(bucket) < nb else 0


def rar_bucket_pack(b: Buckets, bucket: int, tensors: Sequence[Sequence], bucket_bufs: Sequence,
                    stream=None) -> None:
    _check_bucket_bufs(b, bucket_bufs, _bucket_elems(b, bucket))
    _check(lib().rar_bucket_pack(b.handle, int(bucket), len(tensors), _rank_major(b, tensors),
                                 _ranks(bucket_bufs, len(tensors), "bucket_bufs"), _stream(stream)),
           "rar_bucket_pack")


def rar_bucket_unpack(b: Buckets, bucket: int, bucket_bufs: Sequence, tensors: Sequence[Sequence],
                      stream=None) -> None:
    _check_bucket_bufs(b, bucket_bufs, _bucket_elems(b, bucket))
    _check(lib().rar_bucket_unpack(b.handle, int(bucket), len(tensors),
                                   _ranks(bucket_bufs, len(tensors), "bucket_bufs"),
                                   _rank_major(b, tensors), _stream(stream)), "rar_bucket_unpack")


def rar_bucket_allreduce_mean(b: Buckets, tensors: Sequence[Sequence], bucket_bufs=None,
                              chunking: int = BALANCED, algo: int = FUSED, stream=None) -> None:
    """bucket_bufs: N buffers of max_bucket_elems, or None when the reduction
    runs straight from the tensors: RAR_ALGO_FUSED at a supported rank count,
    RAR_ALGO_RING on binary32 at N >= 2, and RAR_ALGO_RING on bf16 when every
    rank's tensors lie end to end in one buffer (see rar.h)."""
    if bucket_bufs is not None and b.handle:
        _check_bucket_bufs(b, bucket_bufs, rar_bucket_count(b)[1])
    bufs = None if bucket_bufs is None else _ranks(bucket_bufs, len(tensors), "bucket_bufs")
    _check(lib().rar_bucket_allreduce_mean(b.handle, len(tensors), int(chunking), int(algo),
                                           _rank_major(b, tensors), bufs, _stream(stream)),
           "rar_bucket_allreduce_mean")


def rar_bucket_allreduce_arena(b: Buckets, arenas: Sequence, ready_events=None, chunking: int = BALANCED,
                               algo: int = FUSED, stream=None) -> None:
    """ready_events: None, or one entry per bucket: a torch.cuda.Event, an
    integer hipEvent_t, or None (no wait)."""
    _check_ranks(arenas, "arenas", b.dtype, b.total)
    ev = None
    if ready_events is not None:
        nb = rar_bucket_count(b)[0]
        if len(ready_events) != nb:
            raise ValueError(f"{len(ready_events)} ready events for {nb} buckets")
        ev = (ctypes.c_void_p * max(len(ready_events), 1))()
        for i, e in enumerate(ready_events):
            ev[i] = None if e is None else (e if isinstance(e, int) else int(e.cuda_event)) or None
    _check(lib().rar_bucket_allreduce_arena(b.handle, len(arenas), int(chunking), int(algo), _ptr_array(arenas),
                                            ev, _stream(stream)), "rar_bucket_allreduce_arena")
