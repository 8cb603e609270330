"""CPU oracle for the ring all-reduce-mean (+ synchronous SGD).

TEST INFRASTRUCTURE ONLY.  Only tests/, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library in ring_all_reduce_amd/) never imports, links or falls back to
it, and the two share no code.

The arithmetic lives in ring_oracle.c (a literal simulation of the ring
schedule, see its header for the passages it follows).  This module is
argument marshalling plus the pieces that are pure host bookkeeping:

* partition / owner:  the chunk table ([Gibiansky] §Scatter-reduce; owner
  derived from the scatter-reduce rule and the all-gather step-1 table).
* ring traffic:       elements each rank sends and receives
  ([Gibiansky] §Allreduce communication cost).
* bucket_layout:      greedy fixed-size buckets over a tensor list given in
  backward order ([Gibiansky] §Applying allreduce to deep learning: the
  reduction may run on a subset of the parameters, output layers first).
* sampled parity:     the literal ring restricted to a sorted subset of
  element indices, which keeps every sampled element in its own chunk.

Short names:
  [Gibiansky]  "Bringing HPC Techniques to Deep Learning" (A. Gibiansky,
               Baidu SVAIL; Korean translation).
  [TrainMGPU]  "[AI System] Training With Multiple GPUs".
  [DDPpage]    "[PyTorch] GPU 분산 학습 1 - DP / DDP / FSDP 개념".

Parity pinned (see tests/test_oracle_pins.py), including the two conventions
the pages leave open.  The mean is one correctly rounded binary32 quotient
S/N, not S*(1/N): pinned by integer inputs whose exact mean is known, and by a
case where the two differ.  The SGD update rounds the product lr*m and then
the difference w - (lr*m), with no fused multiply-add: pinned by hand-derived
cases that tell the two apart and by an element-wise check against exact
rational arithmetic.
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Sequence

import numpy as np

BALANCED, CEIL, ALIGN16 = 0, 1, 2

_HERE = pathlib.Path(__file__).resolve().parent
_LIB = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)


class OracleError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libring_oracle.so, compiling it first if it is not there."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = _HERE / "libring_oracle.so"
    if not path.exists():
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(str(path))
    L.oracle_partition.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _i64p]
    L.oracle_ring_f32.argtypes = [ctypes.c_int, _i64p, ctypes.POINTER(_f32p), _f32p, ctypes.c_float,
                                  _i64p, _i64p]
    L.oracle_ring_f32_ex.argtypes = [ctypes.c_int, _i64p, ctypes.POINTER(_f32p), _f32p,
                                     ctypes.c_float, _i64p, _i64p, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int32)]
    L.oracle_ring_bf16.argtypes = [ctypes.c_int, _i64p, ctypes.POINTER(_u16p), ctypes.POINTER(_u16p),
                                   _f32p, ctypes.c_float, _i64p, _i64p]
    L.oracle_naive_f32.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.POINTER(_f32p), _f32p,
                                   ctypes.c_float, _i64p, _i64p]
    L.oracle_f32_to_bf16_array.argtypes = [_f32p, _u16p, ctypes.c_int64]
    L.oracle_bf16_to_f32_array.argtypes = [_u16p, _f32p, ctypes.c_int64]
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_get_threads.restype = ctypes.c_int
    _LIB = L
    return L


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


def set_threads(t: int) -> None:
    lib().oracle_set_threads(int(t))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


# --------------------------------------------------------------------------
# Chunk table
# --------------------------------------------------------------------------

def partition(N: int, P: int, mode: int = BALANCED, elem_bytes: int = 4) -> np.ndarray:
    """Chunk offsets off[0..N]; chunk c is [off[c], off[c+1])."""
    off = np.zeros(N + 1, dtype=np.int64)
    _check(lib().oracle_partition(int(N), int(P), int(mode), int(elem_bytes), _ptr(off, _i64p)),
           "partition")
    return off


def owner(c: int, N: int) -> int:
    """Rank that holds the finished chunk c after scatter-reduce.

    Derived: at step N-2 rank n sends chunk n+2 to rank n+1, so rank m ends
    with chunk m+1; the all-gather step-1 table of [Gibiansky] (GPU n starts
    by sending chunk n+1) confirms it."""
    return (c - 1) % N


# --------------------------------------------------------------------------
# The literal ring
# --------------------------------------------------------------------------

def _as_ptr_array(arrays: Sequence[np.ndarray], typ):
    arr = (typ * len(arrays))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data_as(typ)
    return arr


def _check_bufs(bufs, dtype, P):
    for b in bufs:
        if b.dtype != dtype or not b.flags["C_CONTIGUOUS"] or b.ndim != 1 or b.shape[0] != P:
            raise OracleError(f"rank buffers must be contiguous 1-D {dtype} of length {P}")


def ring_allreduce_f32(bufs: Sequence[np.ndarray], off: np.ndarray, w: np.ndarray | None = None,
                       lr: float = 0.0):
    """In place over the N float32 rank buffers (and w when given).

    Returns (sent, recv): elements each rank sent and received."""
    N = len(bufs)
    off = np.ascontiguousarray(off, dtype=np.int64)
    P = int(off[N])
    _check_bufs(bufs, np.float32, P)
    if w is not None:
        _check_bufs([w], np.float32, P)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    rc = lib().oracle_ring_f32(N, _ptr(off, _i64p), _as_ptr_array(bufs, _f32p),
                               _ptr(w, _f32p) if w is not None else None, ctypes.c_float(0.0 if lr is None else lr),
                               _ptr(sent, _i64p), _ptr(recv, _i64p))
    _check(rc, "oracle_ring_f32")
    return sent, recv


def ring_partial_f32(bufs: Sequence[np.ndarray], off: np.ndarray, sr_steps: int = -1,
                     ag_steps: int = -1, w: np.ndarray | None = None, lr: float = 0.0):
    """The literal ring cut short after sr_steps scatter-reduce steps (then no
    mean and no all-gather) or after ag_steps all-gather steps, in place.

    Returns (sent, recv, trace) where trace is an (T, 4) int32 array of the
    transfers made, in order: phase (0 scatter-reduce, 1 all-gather), step,
    sender rank, chunk.  The receiver of every transfer is sender + 1 mod N."""
    N = len(bufs)
    off = np.ascontiguousarray(off, dtype=np.int64)
    P = int(off[N])
    _check_bufs(bufs, np.float32, P)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    trace = np.full((2 * N * max(N - 1, 0), 4), -1, dtype=np.int32)
    rc = lib().oracle_ring_f32_ex(N, _ptr(off, _i64p), _as_ptr_array(bufs, _f32p),
                                  _ptr(w, _f32p) if w is not None else None, ctypes.c_float(0.0 if lr is None else lr),
                                  _ptr(sent, _i64p), _ptr(recv, _i64p), int(sr_steps),
                                  int(ag_steps), trace.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _check(rc, "oracle_ring_f32_ex")
    return sent, recv, trace[trace[:, 0] >= 0]


def ring_traffic(N: int, off: np.ndarray):
    """Schedule-only run of the ring: (sent, recv) element counts per rank."""
    off = np.ascontiguousarray(off, dtype=np.int64)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    _check(lib().oracle_ring_f32(N, _ptr(off, _i64p), None, None, ctypes.c_float(0.0),
                                 _ptr(sent, _i64p), _ptr(recv, _i64p)), "oracle_ring_f32")
    return sent, recv


def ring_allreduce_bf16(bufs: Sequence[np.ndarray], off: np.ndarray, w: np.ndarray | None = None,
                        lr: float = 0.0):
    """In place over N uint16 arrays holding bfloat16 bit patterns."""
    N = len(bufs)
    off = np.ascontiguousarray(off, dtype=np.int64)
    P = int(off[N])
    _check_bufs(bufs, np.uint16, P)
    if w is not None:
        _check_bufs([w], np.float32, P)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    ptrs = _as_ptr_array(bufs, _u16p)
    rc = lib().oracle_ring_bf16(N, _ptr(off, _i64p), ptrs, ptrs,
                                _ptr(w, _f32p) if w is not None else None, ctypes.c_float(0.0 if lr is None else lr),
                                _ptr(sent, _i64p), _ptr(recv, _i64p))
    _check(rc, "oracle_ring_bf16")
    return sent, recv


def naive_reduce_f32(bufs: Sequence[np.ndarray], w: np.ndarray | None = None, lr: float = 0.0):
    """Single-reducer baseline (prior art), in place.  Returns (sent, recv)."""
    N = len(bufs)
    P = int(bufs[0].shape[0]) if N else 0
    _check_bufs(bufs, np.float32, P)
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    rc = lib().oracle_naive_f32(N, P, _as_ptr_array(bufs, _f32p),
                                _ptr(w, _f32p) if w is not None else None, ctypes.c_float(0.0 if lr is None else lr),
                                _ptr(sent, _i64p), _ptr(recv, _i64p))
    _check(rc, "oracle_naive_f32")
    return sent, recv


def naive_traffic(N: int, P: int):
    sent = np.zeros(N, dtype=np.int64)
    recv = np.zeros(N, dtype=np.int64)
    _check(lib().oracle_naive_f32(N, P, None, None, ctypes.c_float(0.0), _ptr(sent, _i64p),
                                  _ptr(recv, _i64p)), "oracle_naive_f32")
    return sent, recv


# --------------------------------------------------------------------------
# bfloat16 conversions
# --------------------------------------------------------------------------

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(x, _f32p), _ptr(y, _u16p), x.size)
    return y


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, dtype=np.float32)
    lib().oracle_bf16_to_f32_array(_ptr(h, _u16p), _ptr(y, _f32p), h.size)
    return y


# --------------------------------------------------------------------------
# Buckets
# --------------------------------------------------------------------------

def bucket_layout(numels: Sequence[int], elem_bytes: int, bucket_bytes: int):
    """Greedy fixed-size buckets over tensors listed in backward order.

    The tensors are laid end to end in the order given; bucket b takes
    elements [b*B, (b+1)*B) of that stream, B = bucket_bytes // elem_bytes,
    and a tensor that crosses a boundary is split.  Returns a list of buckets;
    each bucket is a list of segments (tensor, offset_in_tensor,
    offset_in_bucket, length)."""
    B = bucket_bytes // elem_bytes
    if B <= 0:
        raise OracleError("bucket smaller than one element")
    buckets = []
    cur = []
    fill = 0
    for t, n in enumerate(numels):
        pos = 0
        while pos < n:
            take = min(n - pos, B - fill)
            cur.append((t, pos, fill, take))
            pos += take
            fill += take
            if fill == B:
                buckets.append(cur)
                cur, fill = [], 0
    if cur:
        buckets.append(cur)
    return buckets


def bucketed_ring_f32(rank_tensors: Sequence[Sequence[np.ndarray]], bucket_bytes: int,
                      mode: int = BALANCED):
    """All-reduce-mean of a per-rank list of float32 tensors, bucket by bucket.

    rank_tensors[n][t] is tensor t of rank n (backward order).  Each bucket is
    packed from the tensors, reduced by the literal ring with its own chunk
    table, and unpacked, in place.  Returns the bucket layout."""
    N = len(rank_tensors)
    numels = [int(t.size) for t in rank_tensors[0]]
    layout = bucket_layout(numels, 4, bucket_bytes)
    for segs in layout:
        size = sum(s[3] for s in segs)
        bufs = [np.empty(size, dtype=np.float32) for _ in range(N)]
        for n in range(N):
            for (t, toff, boff, ln) in segs:
                bufs[n][boff:boff + ln] = rank_tensors[n][t].reshape(-1)[toff:toff + ln]
        ring_allreduce_f32(bufs, partition(N, size, mode, 4))
        for n in range(N):
            for (t, toff, boff, ln) in segs:
                rank_tensors[n][t].reshape(-1)[toff:toff + ln] = bufs[n][boff:boff + ln]
    return layout


# --------------------------------------------------------------------------
# Sampled parity at sizes the full simulation would not fit
# --------------------------------------------------------------------------

def compact_layout(off: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Chunk table of the sub-array made of the sorted element indices idx."""
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size and np.any(np.diff(idx) <= 0):
        raise OracleError("sample indices must be strictly increasing")
    return np.searchsorted(idx, np.asarray(off, dtype=np.int64), side="left").astype(np.int64)
