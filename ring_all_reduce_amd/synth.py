"""Seeded synthetic inputs: gradient vectors, weights and tensor-list shapes.

This module holds no arithmetic of the all-reduce itself (no chunking, no
reduction order, no mean, no update, no bucketing).  It only draws the inputs
that both the HIP path and the CPU oracle are fed, so that neither side
produces the other's inputs.  Values are drawn with torch generators on the
requested device; a caller that needs them on the host copies them there.

Workloads follow the shapes on the pages (short names as elsewhere):
  * ResNet-18-sized flat gradient, 11.7M parameters
    ([TrainMGPU] §Memory & Delay, ResNet-18 example).
  * A 300M-parameter speech model, 4 bytes per parameter
    ([Gibiansky] §The communication problem).
  * The Transformer of the GPipe explainer, d=2048, h=8192, V=32000, with
    per-layer Q,K,V,O, two FFN matrices, their biases and two LayerNorms
    ([GPipe explainer] §1, the parameter-count fit P(L)).
  * A 40-rank bf16 case with heavy-tailed (Student-t, 3 degrees of freedom)
    values.  The pages fix no bf16 workload; this one exercises bf16
    storage with binary32 accumulation at a large rank count.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import torch

# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Workload:
    key: int                 # seed family: rank r draws with seed 1000*key + r, w with 1000*key + 999
    name: str
    N: int
    P: int                   # elements per rank (flat workloads)
    dtype: str               # "f32" or "bf16"
    dist: str                # "normal" or "student_t3"
    scale: float             # standard deviation (normal) or multiplier (Student-t)
    lr: Optional[float]      # None: mean only, no SGD
    w_range: Optional[Tuple[float, float]] = None
    layers: int = 0          # > 0: ragged Transformer tensor list instead of a flat vector
    bucket_bytes: int = 0


WORKLOADS = {
    1: Workload(1, "n4_p1000003_f32_mean", 4, 1_000_003, "f32", "normal", 1.0, None),
    2: Workload(2, "n10_resnet18_f32_sgd", 10, 11_700_000, "f32", "normal", 0.01, 0.1, (-0.05, 0.05)),
    3: Workload(3, "n10_p300m_f32_sgd", 10, 300_000_000, "f32", "normal", 1e-3, 1e-3, (-0.05, 0.05)),
    4: Workload(4, "n8_transformer12_f32_bucketed", 8, 735_371_264, "f32", "normal", 1e-3, None,
                None, layers=12, bucket_bytes=25_000_000),
    5: Workload(5, "n40_p100m_bf16_sgd", 40, 100_000_000, "bf16", "student_t3", 1e-3, 1e-4,
                (-0.02, 0.02)),
}


def seed_for(key: int, rank: int) -> int:
    return 1000 * key + rank


def weight_seed(key: int) -> int:
    return 1000 * key + 999


# --------------------------------------------------------------------------
# Draws
# --------------------------------------------------------------------------

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_f32(P: int, seed: int, std: float, device="cpu", out: Optional[torch.Tensor] = None):
    """P float32 values drawn from N(0, std^2)."""
    g = _gen(seed, device)
    t = out if out is not None else torch.empty(P, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=g)
    return t


def student_t3_bf16(P: int, seed: int, scale: float, device="cpu"):
    """P bfloat16 values: scale * z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), four
    independent standard normals per value (a Student-t draw with three
    degrees of freedom), converted to bfloat16 by torch."""
    g = _gen(seed, device)
    z = torch.randn(4, P, dtype=torch.float32, device=device, generator=g)
    chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
    t = z[0] / torch.sqrt(chi) * scale
    del z, chi
    return t.to(torch.bfloat16)


def uniform_f32(P: int, seed: int, lo: float, hi: float, device="cpu"):
    g = _gen(seed, device)
    t = torch.empty(P, dtype=torch.float32, device=device)
    t.uniform_(lo, hi, generator=g)
    return t


def _rank_draw(wl: Workload, r: int, P: int, device):
    s = seed_for(wl.key, r)
    if wl.dist == "normal":
        t = normal_f32(P, s, wl.scale, device)
        return t if wl.dtype == "f32" else t.to(torch.bfloat16)
    if wl.dist == "student_t3":
        t = student_t3_bf16(P, s, wl.scale, device)
        return t if wl.dtype == "bf16" else t.float()
    raise ValueError(wl.dist)


def rank_gradients(wl: Workload, device="cpu", P: Optional[int] = None, N: Optional[int] = None):
    """The N per-rank flat gradients of a workload (optionally at another P/N)."""
    P = wl.P if P is None else P
    N = wl.N if N is None else N
    return [_rank_draw(wl, r, P, device) for r in range(N)]


def pool_elements(wl: Workload, stride_bytes: int, P: Optional[int] = None, N: Optional[int] = None) -> int:
    """Elements of wl's dtype that N ranks of P elements, stride_bytes apart, span."""
    P = wl.P if P is None else P
    N = wl.N if N is None else N
    es = 4 if wl.dtype == "f32" else 2
    return max(1, (N - 1) * stride_bytes // es + P)


def rank_gradients_in_pool(wl: Workload, stride_bytes: int, device="cpu", P: Optional[int] = None,
                           N: Optional[int] = None, pool: Optional[torch.Tensor] = None):
    """The same values as rank_gradients, placed in one allocation: rank n's
    buffer starts n * stride_bytes after the first (a layout choice only; the
    stride is the caller's, e.g. the library's recommendation).  `pool`, if
    given, is used instead of a new allocation (1-D, of wl's dtype, at least
    pool_elements long).  Returns the N views; they keep the pool alive."""
    P = wl.P if P is None else P
    N = wl.N if N is None else N
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    es = 4 if wl.dtype == "f32" else 2
    if stride_bytes % es or stride_bytes < P * es:
        raise ValueError("stride must hold one rank's buffer in whole elements")
    need = pool_elements(wl, stride_bytes, P, N)
    if pool is None:
        pool = torch.empty(need, dtype=dt, device=device)
    elif pool.dtype != dt or pool.dim() != 1 or pool.numel() < need:
        raise ValueError(f"pool must be 1-D {dt} of at least {need} elements")
    views = []
    for r in range(N):
        v = pool[r * stride_bytes // es: r * stride_bytes // es + P]
        v.copy_(_rank_draw(wl, r, P, device))
        views.append(v)
    return views


def weights(wl: Workload, device="cpu", P: Optional[int] = None):
    P = wl.P if P is None else P
    lo, hi = wl.w_range if wl.w_range else (-0.05, 0.05)
    return uniform_f32(P, weight_seed(wl.key), lo, hi, device)


# --------------------------------------------------------------------------
# Transformer tensor list (shapes only)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


def transformer_tensors(layers: int = 12, d: int = 2048, h: int = 8192, V: int = 32000,
                        order: str = "backward") -> List[TensorSpec]:
    """Parameter tensors of the GPipe explainer's Transformer.

    Per layer: LayerNorm 1 (gamma, beta), Q, K, V, O (d x d) with biases,
    LayerNorm 2, FFN d->h and h->d with biases.  Plus the input embedding
    (V x d) and the output softmax (d x V).  order="backward" lists them as
    back-propagation produces them: softmax first, then layers from the last
    to the first (each in reverse), then the embedding."""
    fwd: List[TensorSpec] = [TensorSpec("embed", (V, d))]
    for l in range(layers):
        p = f"layer{l}."
        fwd += [TensorSpec(p + "ln1.gamma", (d,)), TensorSpec(p + "ln1.beta", (d,)),
                TensorSpec(p + "Wq", (d, d)), TensorSpec(p + "bq", (d,)),
                TensorSpec(p + "Wk", (d, d)), TensorSpec(p + "bk", (d,)),
                TensorSpec(p + "Wv", (d, d)), TensorSpec(p + "bv", (d,)),
                TensorSpec(p + "Wo", (d, d)), TensorSpec(p + "bo", (d,)),
                TensorSpec(p + "ln2.gamma", (d,)), TensorSpec(p + "ln2.beta", (d,)),
                TensorSpec(p + "W1", (d, h)), TensorSpec(p + "b1", (h,)),
                TensorSpec(p + "W2", (h, d)), TensorSpec(p + "b2", (d,))]
    fwd.append(TensorSpec("softmax", (d, V)))
    if order == "forward":
        return fwd
    if order == "backward":
        return list(reversed(fwd))
    raise ValueError(order)


def transformer_rank_tensors(wl: Workload, device="cpu", layers: Optional[int] = None,
                             d: int = 2048, h: int = 8192, V: int = 32000,
                             pool: Optional[torch.Tensor] = None, stride_bytes: int = 0):
    """Per-rank gradient tensors (backward order) for the bucketed workload,
    each rank drawing one stream of N(0, scale^2) values split into tensors.
    Each rank's tensors are views of one flat arena: its own allocation, or,
    with `pool` (1-D float32), the slice starting at rank * stride_bytes."""
    specs = transformer_tensors(wl.layers if layers is None else layers, d, h, V)
    total = sum(s.numel for s in specs)
    if pool is not None and (stride_bytes % 4 or stride_bytes < 4 * total or pool.dtype != torch.float32
                             or pool.numel() < (wl.N - 1) * stride_bytes // 4 + total):
        raise ValueError("pool must be float32 and hold N arenas stride_bytes apart")
    ranks = []
    for r in range(wl.N):
        flat = normal_f32(total, seed_for(wl.key, r), wl.scale, device)
        if pool is not None:  # drawn on its own, then placed: the same values either way
            flat = pool[r * stride_bytes // 4: r * stride_bytes // 4 + total].copy_(flat)
        ts, pos = [], 0
        for s in specs:
            ts.append(flat[pos:pos + s.numel].view(s.shape))
            pos += s.numel
        ranks.append((flat, ts))
    return specs, ranks
