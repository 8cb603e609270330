"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Binary32 results must be bit-identical to the oracle (same ring order, same
IEEE operations).  bf16 results must be bit-identical to the oracle's bf16
variant and within 1e-2 of a float64 mean (max |error| / max |mean|).  Small
and ragged cases run the oracle in full.  The full-size workloads are checked
twice: on sampled elements (every chunk boundary +-9 and 10^6 random ones)
through the oracle's literal ring restricted to those elements, plus
whole-array properties (all ranks identical); and on every element of every
rank, in the benchmark's layout and launch shape, against the oracle run over
the whole workload.
"""
import pathlib

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_amd import api, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _host_f32(N, P, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal(P) * scale).astype(np.float32) for _ in range(N)]


def _host_bf16(N, P, seed, scale=1e-3):
    # Student-t(3) draws rounded to bf16 by torch (input generation only)
    return [synth.student_t3_bf16(P, seed * 1000 + r, scale, "cpu").view(torch.int16).numpy().view(np.uint16)
            for r in range(N)]


def _to_dev(arrs):
    return [torch.from_numpy(a.copy()).to(DEV) for a in arrs]


def _bf16_dev(arrs):
    return [torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16) for a in arrs]


def _bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _first_diff(a, b):
    d = np.flatnonzero(a != b)
    return int(d[0]) if d.size else None


def _assert_bits(got, ref, what):
    if got.tobytes() != ref.tobytes():
        nan = np.isnan(ref) if ref.dtype == np.float32 else None
        if nan is not None and np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan]):
            return  # NaN payloads are not part of the contract
        i = _first_diff(got, ref)
        raise AssertionError(f"{what}: first difference at {i}: got {got[i]!r} expected {ref[i]!r}")


F32_CASES = [(1, 1), (1, 1001), (2, 1), (2, 2), (2, 9), (3, 5), (4, 3), (8, 7), (5, 4097), (7, 16),
             (4, 1_000_003), (13, 100_003), (40, 12_345), (64, 1), (64, 1000), (64, 65_539)]


@pytest.mark.parametrize("N,P", F32_CASES)
@pytest.mark.parametrize("mode", [api.BALANCED, api.CEIL, api.ALIGN16])
@pytest.mark.parametrize("algo", [api.FUSED, api.RING, api.NAIVE])
def test_f32_mean_and_sgd_bit_exact(N, P, mode, algo):
    g = _host_f32(N, P, 1000 + N * 7 + P % 1000)
    w0 = np.random.default_rng(5).uniform(-0.05, 0.05, P).astype(np.float32)
    for sgd in (False, True):
        d = _to_dev(g)
        wd = torch.from_numpy(w0.copy()).to(DEV)
        plan = api.rar_plan(N, P, api.F32, mode)
        api.rar_plan_set_algo(plan, algo)
        if sgd:
            api.rar_allreduce_sgd(plan, d, wd, 0.1, P)
        else:
            api.rar_allreduce_mean(plan, d, P)
        torch.cuda.synchronize()
        ref = [x.copy() for x in g]
        wr = w0.copy()
        if algo == api.NAIVE:
            oracle.naive_reduce_f32(ref, wr if sgd else None, 0.1)
        else:
            oracle.ring_allreduce_f32(ref, oracle.partition(N, P, mode, 4), wr if sgd else None, 0.1)
        for n in range(N):
            _assert_bits(d[n].cpu().numpy(), ref[n], f"rank {n} sgd={sgd}")
        if sgd:
            _assert_bits(wd.cpu().numpy(), wr, "weights")


BF16_CASES = [(1, 9), (2, 17), (3, 1001), (8, 8), (8, 1_000_003), (40, 100_007), (64, 777), (5, 3)]


@pytest.mark.parametrize("N,P", BF16_CASES)
@pytest.mark.parametrize("mode", [api.BALANCED, api.CEIL, api.ALIGN16])
@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_bf16_bit_exact_and_within_tolerance(N, P, mode, algo):
    g = _host_bf16(N, P, 77 + N + P % 97)
    w0 = np.random.default_rng(6).uniform(-0.02, 0.02, P).astype(np.float32)
    for sgd in (False, True):
        d = _bf16_dev(g)
        wd = torch.from_numpy(w0.copy()).to(DEV)
        plan = api.rar_plan(N, P, api.BF16, mode)
        api.rar_plan_set_algo(plan, algo)
        if sgd:
            api.rar_allreduce_sgd(plan, d, wd, 1e-4, P)
        else:
            api.rar_allreduce_mean(plan, d, P)
        torch.cuda.synchronize()
        ref = [x.copy() for x in g]
        wr = w0.copy()
        oracle.ring_allreduce_bf16(ref, oracle.partition(N, P, mode, 2), wr if sgd else None, 1e-4)
        for n in range(N):
            got = _bits16(d[n])
            assert got.tobytes() == ref[n].tobytes(), f"rank {n}: first diff {_first_diff(got, ref[n])}"
        if sgd:
            _assert_bits(wd.cpu().numpy(), wr, "weights")
        exact = np.stack([oracle.bf16_to_f32(x) for x in g]).astype(np.float64).sum(0) / N
        y = oracle.bf16_to_f32(_bits16(d[0])).astype(np.float64)
        if np.max(np.abs(exact)) > 0:
            assert np.max(np.abs(y - exact)) / np.max(np.abs(exact)) <= 1e-2


def test_resnet18_sized_sgd_all_algorithms():
    wl = synth.WORKLOADS[2]
    N, P = wl.N, wl.P
    g = [t.cpu().numpy() for t in synth.rank_gradients(wl, "cpu")]
    w0 = synth.weights(wl, "cpu").numpy()
    ref = [x.copy() for x in g]
    wr = w0.copy()
    oracle.ring_allreduce_f32(ref, oracle.partition(N, P), wr, wl.lr)
    for algo in (api.FUSED, api.RING):
        d = _to_dev(g)
        wd = torch.from_numpy(w0.copy()).to(DEV)
        plan = api.rar_plan(N, P)
        api.rar_plan_set_algo(plan, algo)
        api.rar_allreduce_sgd(plan, d, wd, wl.lr, P)
        torch.cuda.synchronize()
        for n in (0, 3, N - 1):
            _assert_bits(d[n].cpu().numpy(), ref[n], f"algo {algo} rank {n}")
        for n in range(1, N):
            assert torch.equal(d[n], d[0])
        _assert_bits(wd.cpu().numpy(), wr, f"algo {algo} weights")


@pytest.mark.parametrize("N,P", [(1, 100), (2, 9), (4, 1_000_003), (10, 123_457), (40, 40_001), (64, 64)])
def test_reduce_scatter_owner_sgd_allgather(N, P):
    g = _host_f32(N, P, 31 + N)
    w0 = np.random.default_rng(2).uniform(-0.05, 0.05, P).astype(np.float32)
    d = _to_dev(g)
    wreps = [torch.from_numpy(w0.copy()).to(DEV) for _ in range(N)]
    plan = api.rar_plan(N, P)
    api.rar_reduce_scatter_sgd_allgather(plan, d, wreps, 0.05, P)
    torch.cuda.synchronize()
    ref = [x.copy() for x in g]
    wr = w0.copy()
    off = oracle.partition(N, P)
    oracle.ring_allreduce_f32(ref, off, wr, 0.05)
    for n in range(N):
        _assert_bits(wreps[n].cpu().numpy(), wr, f"replica {n}")
    for c in range(N):
        o = oracle.owner(c, N)
        _assert_bits(d[o].cpu().numpy()[off[c]:off[c + 1]], ref[o][off[c]:off[c + 1]], f"owner of chunk {c}")


@pytest.mark.parametrize("grid", [1, 2, 7, 64, 1000, 0])
def test_results_do_not_depend_on_launch_shape(grid):
    N, P = 4, 1_000_003
    g = _host_f32(N, P, 4)
    ref = [x.copy() for x in g]
    oracle.ring_allreduce_f32(ref, oracle.partition(N, P))
    for algo in (api.FUSED, api.RING):
        for rep in range(3):
            d = _to_dev(g)
            plan = api.rar_plan(N, P)
            api.rar_plan_set_algo(plan, algo)
            api.rar_plan_set_grid(plan, grid)
            api.rar_allreduce_mean(plan, d, P)
            torch.cuda.synchronize()
            for n in range(N):
                _assert_bits(d[n].cpu().numpy(), ref[n], f"grid {grid} algo {algo} rep {rep} rank {n}")


def test_special_values():
    N, P = 6, 40_009
    g = _host_f32(N, P, 9)
    off = oracle.partition(N, P)
    for c in range(1, N):
        g[c % N][off[c]] = np.inf
        g[(c + 1) % N][off[c] - 1] = np.nan
        g[c % N][off[c] + 1] = np.float32(3e-45)  # subnormal
        g[(c + 2) % N][off[c] + 2] = -np.inf
        g[(c + 3) % N][off[c] + 2] = np.inf  # inf - inf
    for algo in (api.FUSED, api.RING):
        d = _to_dev(g)
        plan = api.rar_plan(N, P)
        api.rar_plan_set_algo(plan, algo)
        api.rar_allreduce_mean(plan, d, P)
        torch.cuda.synchronize()
        ref = [x.copy() for x in g]
        oracle.ring_allreduce_f32(ref, off)
        for n in range(N):
            _assert_bits(d[n].cpu().numpy(), ref[n], f"algo {algo} rank {n}")


# The SGD rounding rule w - fl(lr * m), two roundings and no fused multiply-add
# ([Gibiansky] §The communication problem; [TrainMGPU] §Training Process, step
# 3), on two cases whose bits are derived by hand in the oracle pins: a single
# rank with g = 3, lr = 0.1f, w = 0.3f gives +0 (an FMA gives 2^-27), and ten
# ranks whose integer gradients sum to 1 with lr = 0.1f, w = 0.01f give the
# mean fl(1/10) = 0x3DCCCCCD and w = -2^-30 = 0xB0800000 (an FMA gives
# 0xB00F5C29).  P spans vector bodies, heads and tails of every chunk.
SGD_HAND_CASES = {
    "one_rank": dict(N=1, grads=[3.0], lr=0.1, w=0.3, mean_bits=0x40400000, bf16_mean=0x4040, w_bits=0x00000000),
    "ten_ranks": dict(N=10, grads=[1.0] * 9 + [-8.0], lr=0.1, w=0.01, mean_bits=0x3DCCCCCD, bf16_mean=0x3DCD,
                      w_bits=0xB0800000),
}


@pytest.mark.parametrize("case", sorted(SGD_HAND_CASES))
@pytest.mark.parametrize("path", ["fused", "ring", "naive", "rs_sgd_ag", "bf16_fused", "bf16_ring"])
def test_sgd_rounding_hand_cases_every_path(case, path):
    c = SGD_HAND_CASES[case]
    N, P, lr = c["N"], 40_013, c["lr"]
    host = [np.full(P, v, np.float32) for v in c["grads"]]
    w0 = np.full(P, c["w"], np.float32)
    if path.startswith("bf16"):
        hb = [oracle.f32_to_bf16(h) for h in host]
        assert all(np.array_equal(oracle.bf16_to_f32(b), h) for b, h in zip(hb, host))  # exact in bf16
        d = _bf16_dev(hb)
        plan = api.rar_plan(N, P, api.BF16)
        api.rar_plan_set_algo(plan, api.FUSED if path == "bf16_fused" else api.RING)
        wd = torch.from_numpy(w0.copy()).to(DEV)
        api.rar_allreduce_sgd(plan, d, wd, lr, P)
        torch.cuda.synchronize()
        ref, wr = [b.copy() for b in hb], w0.copy()
        oracle.ring_allreduce_bf16(ref, oracle.partition(N, P, api.BALANCED, 2), wr, lr)
        for n in range(N):
            got = _bits16(d[n])
            assert np.all(got == c["bf16_mean"]), f"rank {n}: {hex(int(got[0]))}"
            assert got.tobytes() == ref[n].tobytes()
        wg = wd.cpu().numpy()
        assert np.all(wg.view(np.uint32) == c["w_bits"]), hex(int(wg.view(np.uint32)[0]))
        assert wg.tobytes() == wr.tobytes()
        return
    d = _to_dev(host)
    plan = api.rar_plan(N, P)
    ref, wr = [h.copy() for h in host], w0.copy()
    if path == "naive":
        oracle.naive_reduce_f32(ref, wr, lr)
    else:
        oracle.ring_allreduce_f32(ref, oracle.partition(N, P), wr, lr)
    if path == "rs_sgd_ag":
        reps = [torch.from_numpy(w0.copy()).to(DEV) for _ in range(N)]
        api.rar_reduce_scatter_sgd_allgather(plan, d, reps, lr, P)
        torch.cuda.synchronize()
        for n, r in enumerate(reps):
            wg = r.cpu().numpy()
            assert np.all(wg.view(np.uint32) == c["w_bits"]), f"replica {n}: {hex(int(wg.view(np.uint32)[0]))}"
            assert wg.tobytes() == wr.tobytes()
        return
    api.rar_plan_set_algo(plan, {"fused": api.FUSED, "ring": api.RING, "naive": api.NAIVE}[path])
    wd = torch.from_numpy(w0.copy()).to(DEV)
    api.rar_allreduce_sgd(plan, d, wd, lr, P)
    torch.cuda.synchronize()
    for n in range(N):
        got = d[n].cpu().numpy()
        assert np.all(got.view(np.uint32) == c["mean_bits"]), f"rank {n}"
        assert got.tobytes() == ref[n].tobytes()
    wg = wd.cpu().numpy()
    assert np.all(wg.view(np.uint32) == c["w_bits"]), hex(int(wg.view(np.uint32)[0]))
    assert wg.tobytes() == wr.tobytes()


def test_runs_on_the_given_stream():
    N, P = 8, 2_000_000
    g = _host_f32(N, P, 12)
    ref = [x.copy() for x in g]
    oracle.ring_allreduce_f32(ref, oracle.partition(N, P))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d = _to_dev(g)
        plan = api.rar_plan(N, P)
        api.rar_allreduce_mean(plan, d, P, stream=s)
    s.synchronize()
    for n in range(N):
        _assert_bits(d[n].cpu().numpy(), ref[n], f"rank {n}")


# ---------------------------------------------------------------------------
# Buckets
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [api.F32, api.BF16])
def test_bucket_pack_unpack_roundtrip_unaligned(dt):
    tdt = torch.float32 if dt == api.F32 else torch.bfloat16
    es = 4 if dt == api.F32 else 2
    numels = [5, 1, 1000, 3, 77, 4096, 2]
    N = 3
    arenas = [torch.randn(sum(numels) + 7, device=DEV).to(tdt) for _ in range(N)]
    tensors, pos = [], 1  # odd start: every tensor misaligned
    for n in range(N):
        ts, p = [], pos
        for k in numels:
            ts.append(arenas[n][p:p + k])
            p += k
        tensors.append(ts)
    b = api.rar_bucket_plan(numels, dt, 96 * es)
    nb, mx = api.rar_bucket_count(b)
    bufs = [torch.zeros(mx, dtype=tdt, device=DEV) for _ in range(N)]
    backup = [a.clone() for a in arenas]
    layout = oracle.bucket_layout(numels, es, 96 * es)
    for k in range(nb):
        api.rar_bucket_pack(b, k, tensors, bufs)
        torch.cuda.synchronize()
        for n in range(N):
            for (t, toff, boff, ln) in layout[k]:
                assert torch.equal(bufs[n][boff:boff + ln], tensors[n][t][toff:toff + ln])
        for n in range(N):
            for (t, toff, boff, ln) in layout[k]:
                tensors[n][t][toff:toff + ln].zero_()
        api.rar_bucket_unpack(b, k, bufs, tensors)
    torch.cuda.synchronize()
    for n in range(N):
        assert torch.equal(arenas[n], backup[n])


def test_bucket_buffers_packed_tightly_beside_the_tensors():
    """Bucket buffers back to back and the tensors right after them in one
    allocation: ranges that only touch pass the overlap checks, and the
    packing path reduces bit-exactly."""
    N = 4
    specs = synth.transformer_tensors(2, d=64, h=256, V=1000)
    numels = [s.numel for s in specs]
    bucket_bytes = 4 * 40_004
    host = [[np.random.default_rng(700 + 100 * n + t).standard_normal(s.numel).astype(np.float32)
             for t, s in enumerate(specs)] for n in range(N)]
    ref = [[x.copy() for x in rank] for rank in host]
    layout = oracle.bucketed_ring_f32(ref, bucket_bytes, api.BALANCED)
    b = api.rar_bucket_plan(numels, api.F32, bucket_bytes)
    nb, mx = api.rar_bucket_count(b)
    total = sum(numels)
    span = -(-mx // 4) * 4                        # whole 16-byte units
    pool = torch.zeros(N * span + N * total, device=DEV)
    bufs = [pool[n * span:(n + 1) * span] for n in range(N)]
    arenas = [pool[N * span + n * total:N * span + (n + 1) * total] for n in range(N)]
    for n in range(N):
        arenas[n].copy_(torch.from_numpy(np.concatenate(host[n])))
    starts = np.concatenate([[0], np.cumsum(numels)])
    tensors = [[a[starts[t]:starts[t + 1]] for t in range(len(numels))] for a in arenas]
    api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, api.RING)
    torch.cuda.synchronize()
    for n in range(N):
        for t in range(len(specs)):
            _assert_bits(tensors[n][t].cpu().numpy(), ref[n][t], f"rank {n} tensor {t}")
    # the last (short) bucket's buffers spaced by its own size only
    k = nb - 1
    ek = api.rar_bucket_info(b, k)[1]
    assert ek < mx
    step = -(-ek // 4) * 4
    small = [pool[n * step:n * step + ek] for n in range(N)]
    api.rar_bucket_pack(b, k, tensors, small)
    torch.cuda.synchronize()
    for n in range(N):
        for (t, toff, boff, ln) in layout[k]:
            assert torch.equal(small[n][boff:boff + ln], tensors[n][t][toff:toff + ln])


@pytest.mark.parametrize("mode", [api.BALANCED, api.CEIL, api.ALIGN16])
@pytest.mark.parametrize("N", [4, 10])
def test_bucketed_small_transformer_bit_exact(N, mode):
    # buckets of 40,004 elements (16-byte multiples, so arena slices stay
    # aligned); at N = 10 the three chunkings cut them differently:
    # balanced 4001 x 4 + 4000 x 6, ceil 4001 x 9 + 3995, align16 4004 x 9 + 3968
    specs = synth.transformer_tensors(2, d=64, h=256, V=1000)
    numels = [s.numel for s in specs]
    bucket_bytes = 4 * 40_004
    host = [[np.random.default_rng(100 * n + t).standard_normal(s.numel).astype(np.float32) * 1e-3
             for t, s in enumerate(specs)] for n in range(N)]
    ref = [[x.copy() for x in rank] for rank in host]
    oracle.bucketed_ring_f32(ref, bucket_bytes, mode)
    b = api.rar_bucket_plan(numels, api.F32, bucket_bytes)
    _, mx = api.rar_bucket_count(b)
    starts = np.concatenate([[0], np.cumsum(numels)])
    for path in ("tensors", "arena", "ring"):
        arenas = [torch.from_numpy(np.concatenate(rank)).to(DEV) for rank in host]
        tensors = [[a[starts[t]:starts[t + 1]] for t in range(len(numels))] for a in arenas]
        if path == "tensors":
            api.rar_bucket_allreduce_mean(b, tensors, None, mode, api.FUSED)
        elif path == "arena":
            api.rar_bucket_allreduce_arena(b, arenas, None, mode, api.FUSED)
        else:
            bufs = [torch.empty(mx, device=DEV) for _ in range(N)]
            api.rar_bucket_allreduce_mean(b, tensors, bufs, mode, api.RING)
        torch.cuda.synchronize()
        for n in range(N):
            for t in range(len(specs)):
                _assert_bits(tensors[n][t].cpu().numpy(), ref[n][t], f"{path} rank {n} tensor {t}")


# ---------------------------------------------------------------------------
# Full-size workloads, sampled
# ---------------------------------------------------------------------------

def _samples(off, P, k, seed):
    rng = np.random.default_rng(seed)
    edges = np.array([o + dlt for o in off for dlt in range(-9, 10)], dtype=np.int64)
    idx = np.unique(np.concatenate([edges, rng.integers(0, P, k)]))
    return idx[(idx >= 0) & (idx < P)]


def _gather(ts, idx_d):
    return [t[idx_d].cpu().numpy() for t in ts]


@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_full_size_300m_sgd_sampled(algo):
    wl = synth.WORKLOADS[3]
    N, P = wl.N, wl.P
    off = oracle.partition(N, P)
    idx = _samples(off, P, 1_000_000, 3)
    idx_d = torch.from_numpy(idx).to(DEV)
    g = synth.rank_gradients(wl, DEV)
    w = synth.weights(wl, DEV)
    pre = _gather(g, idx_d)
    wpre = w[idx_d].cpu().numpy()
    plan = api.rar_plan(N, P)
    api.rar_plan_set_algo(plan, algo)
    api.rar_allreduce_sgd(plan, g, w, wl.lr, P)
    torch.cuda.synchronize()
    for n in range(1, N):
        assert torch.equal(g[n], g[0]), f"rank {n} differs from rank 0"
    oracle.ring_allreduce_f32(pre, oracle.compact_layout(off, idx), wpre, wl.lr)
    post = _gather(g, idx_d)
    for n in (0, N - 1):
        _assert_bits(post[n], pre[n], f"rank {n} (sampled)")
    _assert_bits(w[idx_d].cpu().numpy(), wpre, "weights (sampled)")


@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_full_size_40_rank_bf16_sampled(algo):
    wl = synth.WORKLOADS[5]
    N, P = wl.N, wl.P
    off = oracle.partition(N, P, 0, 2)
    idx = _samples(off, P, 500_000, 5)
    idx_d = torch.from_numpy(idx).to(DEV)
    g = synth.rank_gradients(wl, DEV)
    w = synth.weights(wl, DEV)
    pre = [_bits16(t[idx_d]) for t in g]
    wpre = w[idx_d].cpu().numpy()
    plan = api.rar_plan(N, P, api.BF16)
    api.rar_plan_set_algo(plan, algo)
    api.rar_allreduce_sgd(plan, g, w, wl.lr, P)
    torch.cuda.synchronize()
    for n in range(1, N):
        assert torch.equal(g[n].view(torch.int16), g[0].view(torch.int16)), f"rank {n} differs"
    exact = np.stack([oracle.bf16_to_f32(x) for x in pre]).astype(np.float64).sum(0) / N
    oracle.ring_allreduce_bf16(pre, oracle.compact_layout(off, idx), wpre, wl.lr)
    post = _bits16(g[0][idx_d])
    assert post.tobytes() == pre[0].tobytes(), f"first diff {_first_diff(post, pre[0])}"
    _assert_bits(w[idx_d].cpu().numpy(), wpre, "weights (sampled)")
    y = oracle.bf16_to_f32(post).astype(np.float64)
    assert np.max(np.abs(y - exact)) / np.max(np.abs(exact)) <= 1e-2


@pytest.mark.parametrize("path", ["tensors", "arena", "tensors_ring"])
def test_full_size_transformer_buckets_sampled(path):
    wl = synth.WORKLOADS[4]
    N = wl.N
    specs, ranks = synth.transformer_rank_tensors(wl, DEV)
    numels = [s.numel for s in specs]
    total = sum(numels)
    arenas = [flat for (flat, _) in ranks]
    tensors = [ts for (_, ts) in ranks]
    b = api.rar_bucket_plan(numels, api.F32, wl.bucket_bytes)
    nb, mx = api.rar_bucket_count(b)
    assert nb == 118
    rng = np.random.default_rng(44)
    per_bucket = []
    for k in range(nb):
        so, el, _ = api.rar_bucket_info(b, k)
        off = oracle.partition(N, el)
        idx = _samples(off, el, 2000, int(rng.integers(1 << 30)))
        per_bucket.append((so, el, off, idx))
    all_idx = np.concatenate([so + idx for (so, _, _, idx) in per_bucket])
    idx_d = torch.from_numpy(all_idx).to(DEV)
    pre = _gather(arenas, idx_d)
    if path == "tensors":  # straight from the tensor lists, no bucket buffers
        api.rar_bucket_allreduce_mean(b, tensors, None)
    elif path == "tensors_ring":  # pack, ring steps, unpack
        bufs = [torch.empty(mx, device=DEV) for _ in range(N)]
        api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, api.RING)
    else:
        plans = {}
        for (so, el, _, _) in per_bucket:
            if el not in plans:
                plans[el] = api.rar_plan(N, el)
            api.rar_allreduce_mean(plans[el], [a[so:so + el] for a in arenas], el)
    torch.cuda.synchronize()
    for n in range(1, N):
        assert torch.equal(arenas[n], arenas[0])
    post = _gather(arenas, idx_d)
    pos = 0
    for (so, el, off, idx) in per_bucket:
        sl = slice(pos, pos + len(idx))
        sub = [np.ascontiguousarray(p[sl]) for p in pre]
        oracle.ring_allreduce_f32(sub, oracle.compact_layout(off, idx))
        _assert_bits(post[0][sl], sub[0], f"bucket at {so}")
        pos += len(idx)
    assert pos == len(all_idx) and total == 735_371_264


# ---------------------------------------------------------------------------
# Largest shapes: element offsets past 2^31, and the maximum rank count
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_offsets_beyond_32_bits_sampled(algo):
    # 2 ranks x (2^31 + 7) binary32 elements: every byte offset of the second
    # half of each buffer exceeds 2^32, element offsets exceed 2^31
    N, P = 2, 2 ** 31 + 7
    off = oracle.partition(N, P)
    idx = _samples(off, P, 200_000, 11)
    idx = np.unique(np.concatenate([idx, np.array([P - 1, P - 2, 2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1])]))
    idx_d = torch.from_numpy(idx).to(DEV)
    g = [synth.normal_f32(P, 500 + r, 1.0, DEV) for r in range(N)]
    w = synth.uniform_f32(P, 599, -0.05, 0.05, DEV)
    pre = _gather(g, idx_d)
    wpre = w[idx_d].cpu().numpy()
    plan = api.rar_plan(N, P)
    api.rar_plan_set_algo(plan, algo)
    api.rar_allreduce_sgd(plan, g, w, 0.01, P)
    torch.cuda.synchronize()
    assert torch.equal(g[0], g[1])
    oracle.ring_allreduce_f32(pre, oracle.compact_layout(off, idx), wpre, 0.01)
    _assert_bits(g[1][idx_d].cpu().numpy(), pre[1], "rank 1 (sampled)")
    _assert_bits(w[idx_d].cpu().numpy(), wpre, "weights (sampled)")


@pytest.mark.parametrize("dt", [api.F32, api.BF16])
def test_sixty_four_ranks_sampled(dt):
    N, P = 64, 10_000_019
    eb = 4 if dt == api.F32 else 2
    off = oracle.partition(N, P, api.BALANCED, eb)
    idx = _samples(off, P, 100_000, 12)
    idx_d = torch.from_numpy(idx).to(DEV)
    g = [synth.normal_f32(P, 700 + r, 1e-2, DEV) for r in range(N)]
    if dt == api.BF16:
        g = [t.to(torch.bfloat16) for t in g]
    w = synth.uniform_f32(P, 799, -0.05, 0.05, DEV)
    pre = [_bits16(t[idx_d]) for t in g] if dt == api.BF16 else _gather(g, idx_d)
    wpre = w[idx_d].cpu().numpy()
    for algo in (api.FUSED, api.RING):
        plan = api.rar_plan(N, P, dt)
        api.rar_plan_set_algo(plan, algo)
        d = [t.clone() for t in g]
        wd = w.clone()
        api.rar_allreduce_sgd(plan, d, wd, 1e-3, P)
        torch.cuda.synchronize()
        ref = [x.copy() for x in pre]
        wr = wpre.copy()
        if dt == api.BF16:
            oracle.ring_allreduce_bf16(ref, oracle.compact_layout(off, idx), wr, 1e-3)
            got = _bits16(d[N - 1][idx_d])
            assert got.tobytes() == ref[N - 1].tobytes(), f"algo {algo}: first diff {_first_diff(got, ref[N - 1])}"
        else:
            oracle.ring_allreduce_f32(ref, oracle.compact_layout(off, idx), wr, 1e-3)
            _assert_bits(d[N - 1][idx_d].cpu().numpy(), ref[N - 1], f"algo {algo} rank {N - 1}")
        _assert_bits(wd[idx_d].cpu().numpy(), wr, f"algo {algo} weights")
        del d, wd


# ---------------------------------------------------------------------------
# Buckets reduced as a simulated backward pass produces them
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [api.F32, api.BF16])
@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_bucket_arena_waits_for_each_ready_event(algo, dt):
    # The producer stream writes bucket k only after a long matrix product, the
    # arenas start as NaN, and the reduction runs on another stream: a reduction
    # that did not wait for bucket k's event would read NaN and fail parity.
    N = 4
    specs = synth.transformer_tensors(2, d=128, h=512, V=4000)
    numels = [s.numel for s in specs]
    total = sum(numels)
    es = 4 if dt == api.F32 else 2
    bucket_bytes = es * 100_000
    host = [np.random.default_rng(900 + n).standard_normal(total).astype(np.float32) * 1e-3 for n in range(N)]
    if dt == api.BF16:
        host = [oracle.f32_to_bf16(h) for h in host]
        pristine = _bf16_dev(host)
        arenas = [torch.full((total,), float("nan"), device=DEV, dtype=torch.bfloat16) for _ in range(N)]
    else:
        pristine = [torch.from_numpy(h.copy()).to(DEV) for h in host]
        arenas = [torch.full((total,), float("nan"), device=DEV) for _ in range(N)]
    b = api.rar_bucket_plan(numels, dt, bucket_bytes)
    nb, _ = api.rar_bucket_count(b)
    infos = [api.rar_bucket_info(b, k) for k in range(nb)]
    a = torch.randn(2048, 2048, device=DEV)
    torch.cuda.synchronize()
    producer, comm = torch.cuda.Stream(), torch.cuda.Stream()
    events = []
    with torch.cuda.stream(producer):
        for (so, el, _) in infos:
            a = torch.matmul(a, a) * 1e-3  # stands in for the backward compute of this bucket
            for n in range(N):
                arenas[n][so:so + el].copy_(pristine[n][so:so + el])
            e = torch.cuda.Event()
            e.record(producer)
            events.append(e)
    api.rar_bucket_allreduce_arena(b, arenas, events, algo=algo, stream=comm)
    comm.synchronize()
    producer.synchronize()
    for n in range(1, N):
        assert torch.equal(arenas[n].view(torch.int16 if dt == api.BF16 else torch.int32),
                           arenas[0].view(torch.int16 if dt == api.BF16 else torch.int32))
    got = arenas[0].cpu().numpy() if dt == api.F32 else _bits16(arenas[0])
    for (so, el, _) in infos:
        part = [np.ascontiguousarray(h[so:so + el]) for h in host]
        if dt == api.F32:
            oracle.ring_allreduce_f32(part, oracle.partition(N, el))
        else:
            oracle.ring_allreduce_bf16(part, oracle.partition(N, el, oracle.BALANCED, 2))
        _assert_bits(got[so:so + el], part[0], f"bucket at {so}")


def test_bucket_arena_without_events_matches_pack_path():
    N = 3
    specs = synth.transformer_tensors(1, d=64, h=256, V=1000)
    numels = [s.numel for s in specs]
    total = sum(numels)
    b = api.rar_bucket_plan(numels, api.F32, 4 * 8_000)
    host = [np.random.default_rng(70 + n).standard_normal(total).astype(np.float32) for n in range(N)]
    arenas = [torch.from_numpy(h.copy()).to(DEV) for h in host]
    for algo in (api.FUSED, api.RING):
        ar = [t.clone() for t in arenas]
        api.rar_bucket_allreduce_arena(b, ar, None, api.BALANCED, algo)
        tensors, pos = [[] for _ in range(N)], 0
        flat = [t.clone() for t in arenas]
        for s in specs:
            for n in range(N):
                tensors[n].append(flat[n][pos:pos + s.numel])
            pos += s.numel
        _, mx = api.rar_bucket_count(b)
        bufs = [torch.empty(mx, device=DEV) for _ in range(N)]
        api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, algo)
        torch.cuda.synchronize()
        for n in range(N):
            assert torch.equal(ar[n], flat[n])
        got = ar[0].cpu().numpy()
        for k in range(api.rar_bucket_count(b)[0]):
            so, el, _ = api.rar_bucket_info(b, k)
            part = [np.ascontiguousarray(h[so:so + el]) for h in host]
            oracle.ring_allreduce_f32(part, oracle.partition(N, el))
            _assert_bits(got[so:so + el], part[0], f"algo {algo} bucket {k}")


@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_bucketed_bf16_small_transformer_bit_exact(algo):
    N = 5
    specs = synth.transformer_tensors(1, d=64, h=256, V=777)
    numels = [s.numel for s in specs]
    bucket_bytes = 2 * 30_000
    host = [[synth.student_t3_bf16(s.numel, 3000 + 100 * n + t, 1e-3, "cpu").view(torch.int16).numpy()
             .view(np.uint16).copy() for t, s in enumerate(specs)] for n in range(N)]
    tensors = [[torch.from_numpy(x.view(np.int16).copy()).to(DEV).view(torch.bfloat16) for x in rank]
               for rank in host]
    b = api.rar_bucket_plan(numels, api.BF16, bucket_bytes)
    nb, mx = api.rar_bucket_count(b)
    bufs = [torch.empty(mx, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
    api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, algo)
    torch.cuda.synchronize()
    layout = oracle.bucket_layout(numels, 2, bucket_bytes)
    assert len(layout) == nb
    for segs in layout:
        size = sum(s[3] for s in segs)
        part = [np.concatenate([host[n][t][toff:toff + ln] for (t, toff, _, ln) in segs]) for n in range(N)]
        oracle.ring_allreduce_bf16(part, oracle.partition(N, size, oracle.BALANCED, 2))
        for n in (0, N - 1):
            got = np.concatenate([_bits16(tensors[n][t][toff:toff + ln]) for (t, toff, _, ln) in segs])
            assert got.tobytes() == part[n].tobytes(), f"rank {n}: first diff {_first_diff(got, part[n])}"


@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
@pytest.mark.parametrize("skew", ["same", "different"])
@pytest.mark.parametrize("dt", [api.F32, api.BF16])
def test_bucket_tensors_direct_with_misaligned_views(skew, dt, algo):
    # Tensors are views at odd element offsets: with the same offset on every
    # rank the direct path runs vector bodies with scalar heads and tails; with
    # different offsets per rank it runs the scalar path.  Both must match the
    # oracle bit for bit.
    N = 4
    tdt = torch.float32 if dt == api.F32 else torch.bfloat16
    es = 4 if dt == api.F32 else 2
    numels = [5, 1000, 3, 4097, 77, 20_000, 1]
    total = sum(numels)
    bucket_bytes = es * 3001
    rng = np.random.default_rng(5)
    if dt == api.F32:
        host = [rng.standard_normal(total).astype(np.float32) for _ in range(N)]
    else:
        host = [oracle.f32_to_bf16(rng.standard_normal(total).astype(np.float32) * 1e-2) for _ in range(N)]
    tensors, keep = [], []
    for n in range(N):
        shift = 1 if skew == "same" else 1 + n
        arena = torch.zeros(total + 16, dtype=tdt, device=DEV)
        src = torch.from_numpy(host[n].view(np.int16) if dt == api.BF16 else host[n]).to(DEV)
        arena[shift:shift + total].copy_(src.view(tdt) if dt == api.BF16 else src)
        keep.append(arena)
        ts, pos = [], shift
        for k in numels:
            ts.append(arena[pos:pos + k])
            pos += k
        tensors.append(ts)
    b = api.rar_bucket_plan(numels, dt, bucket_bytes)
    # binary32 ring steps run on the tensor pieces directly; bf16 ring steps pack
    bufs = [torch.empty(api.rar_bucket_count(b)[1], dtype=tdt, device=DEV) for _ in range(N)] \
        if algo == api.RING else None
    api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, algo)
    torch.cuda.synchronize()
    layout = oracle.bucket_layout(numels, es, bucket_bytes)
    stream = [h.copy() for h in host]
    pos = 0
    for segs in layout:
        size = sum(sg[3] for sg in segs)
        part = [np.ascontiguousarray(h[pos:pos + size]) for h in stream]
        if dt == api.F32:
            oracle.ring_allreduce_f32(part, oracle.partition(N, size))
        else:
            oracle.ring_allreduce_bf16(part, oracle.partition(N, size, oracle.BALANCED, 2))
        for n in range(N):
            stream[n][pos:pos + size] = part[n]
        pos += size
    for n in range(N):
        shift = 1 if skew == "same" else 1 + n
        got = keep[n][shift:shift + total]
        got = _bits16(got) if dt == api.BF16 else got.cpu().numpy()
        assert got.tobytes() == stream[n].tobytes(), f"rank {n}: first diff {_first_diff(got, stream[n])}"


def test_hundred_repeats_with_varied_launch_shapes_are_identical():
    # race check: 100 runs from the same inputs with workgroup caps drawn at
    # random (grid-stride loops of every length) must give identical bits
    N, P = 4, 1_000_003
    g = _host_f32(N, P, 21)
    pristine = [torch.from_numpy(x).to(DEV) for x in g]
    w0 = torch.linspace(-0.05, 0.05, P, device=DEV)
    ref = [x.copy() for x in g]
    wr = w0.cpu().numpy().copy()
    oracle.ring_allreduce_f32(ref, oracle.partition(N, P), wr, 0.1)
    rng = np.random.default_rng(99)
    for rep in range(100):
        algo = api.FUSED if rep % 2 == 0 else api.RING
        d = [t.clone() for t in pristine]
        wd = w0.clone()
        plan = api.rar_plan(N, P)
        api.rar_plan_set_algo(plan, algo)
        api.rar_plan_set_grid(plan, int(rng.choice([0, 1, 3, 17, 64, 255, 1024, 5000])))
        api.rar_allreduce_sgd(plan, d, wd, 0.1, P)
        torch.cuda.synchronize()
        for n in (0, N - 1):
            assert d[n].cpu().numpy().tobytes() == ref[n].tobytes(), f"rep {rep} algo {algo} rank {n}"
        assert wd.cpu().numpy().tobytes() == wr.tobytes(), f"rep {rep} weights"


@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_bf16_special_values(algo):
    # bf16 infinities, NaN, subnormals and values whose mean rounds to the
    # largest finite bf16 or overflows to infinity, placed at chunk heads,
    # tails and bodies.
    N, P = 4, 8 * 1000 + 5
    rng = np.random.default_rng(3)
    g = [oracle.f32_to_bf16(rng.standard_normal(P).astype(np.float32)) for _ in range(N)]
    off = oracle.partition(N, P, api.BALANCED, 2)
    specials = [0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8001, 0x0080, 0x7F7F, 0xFF7F]
    for c in range(N):
        for i, s in enumerate(specials):
            e = int(off[c]) + i * 3
            g[(c + i) % N][e] = s
        for r in range(N):
            g[r][int(off[c]) + 40] = 0x7F7F  # four bf16 maxima overflow binary32: the mean is infinity
            g[r][int(off[c]) + 41] = 0x0001  # smallest subnormal everywhere
    w0 = np.zeros(P, np.float32)
    d = _bf16_dev(g)
    wd = torch.from_numpy(w0.copy()).to(DEV)
    plan = api.rar_plan(N, P, api.BF16)
    api.rar_plan_set_algo(plan, algo)
    api.rar_allreduce_sgd(plan, d, wd, 1e-3, P)
    torch.cuda.synchronize()
    ref = [x.copy() for x in g]
    wr = w0.copy()
    oracle.ring_allreduce_bf16(ref, off, wr, 1e-3)
    for n in range(N):
        got = _bits16(d[n])
        gf, rf = oracle.bf16_to_f32(got), oracle.bf16_to_f32(ref[n])
        nan = np.isnan(rf)
        assert np.array_equal(np.isnan(gf), nan), f"rank {n}: NaN positions differ"
        assert got[~nan].tobytes() == ref[n][~nan].tobytes(), f"rank {n}: first diff {_first_diff(got, ref[n])}"
    _assert_bits(wd.cpu().numpy(), wr, "weights")


def _bf16_rounding_cases(N):
    """bf16 rank inputs (N in {2, 4}) whose binary32 mean lands on chosen
    bit patterns, and a label per element.  Every sum is exact in any order
    (at most one NaN per element), so the mean does not depend on the fold.

    - "tie": the mean is exactly halfway between two bf16 values, at every
      binary32 exponent whose partial sums stay finite, with the kept bit even and
      odd, and with the kept bits all ones (the rounding carries into the
      exponent); and every subnormal tie.  The tie 0x7F7F8000, which would
      round to infinity, cannot be a mean of N >= 2 finite inputs: its sum
      would exceed the binary32 range.
    - "near": dropped bits 0x4000 and 0xC000 (round down, round up).
    - "overflow": the sum overflows, so the mean is infinity.
    - "nan": one rank holds a quiet or signalling NaN with a payload.
    Ranks: N = 2 holds (a, b); N = 4 holds (a, b, b, -b), whose sum is a + b.
    """
    assert N in (2, 4)
    lg = N.bit_length() - 1
    ops, kinds = [], []

    def add(a, b, kind):
        vals = [a, b] if N == 2 else [a, b, b, -b]
        v32 = np.array(vals, np.float32)
        assert np.array_equal(v32.astype(np.float64), np.array(vals)), vals
        h = oracle.f32_to_bf16(v32)
        assert np.array_equal(oracle.bf16_to_f32(h), v32), vals  # exact in bf16
        ops.append(h)
        kinds.append(kind)

    # N = 4 folds a + b + b in some chunks: a + 2b = 2^(e+3) at k = 0x7F must
    # stay finite, so e <= 124 there; N = 2 only forms a + b, so e <= 126
    for e in range(-126, 125 if N == 4 else 127):
        for k in (0, 1, 0x2A, 0x55, 0x7E, 0x7F):
            a = N * 2.0 ** e * (1 + k / 128)
            b = N * 2.0 ** (e - 8)
            m = np.float32(np.float32(a) + np.float32(b)) / np.float32(N)
            assert int(m.view(np.uint32)) == ((e + 127) << 23) | (k << 16) | 0x8000
            add(a, b, "tie")
        if e % 17 == 0:
            a = N * 2.0 ** e * (1 + 0x33 / 128)
            add(a, 1.5 * N * 2.0 ** (e - 8), "near")   # dropped 0xC000: rounds up
            add(a, -1.5 * N * 2.0 ** (e - 8), "near")  # 0x33 - 1 kept, dropped 0x4000: rounds down
    for k in range(128):  # subnormal ties: m = (k << 16 | 0x8000) * 2^-149
        b = (N // 2) * 2.0 ** -133
        a = k * N * 2.0 ** -133
        m = np.float32(np.float32(a) + np.float32(b)) / np.float32(N)
        assert int(m.view(np.uint32)) == (k << 16) | 0x8000
        add(a, b, "tie")
    bmax = float(oracle.bf16_to_f32(np.array([0x7F7F], np.uint16))[0])
    add(bmax, bmax, "overflow")
    for p in (0x7FC1, 0x7F81, 0xFFA5, 0x7FFF, 0xFFC0):
        for r in range(N):
            h = oracle.f32_to_bf16(np.ones(N, np.float32))
            h[r] = p
            ops.append(h)
            kinds.append("nan")
    return np.stack(ops), np.array(kinds)


@pytest.mark.parametrize("N", [2, 4])
@pytest.mark.parametrize("path", ["fused", "ring", "bucket_tensors", "bucket_ring"])
def test_bf16_narrowing_ties_and_nan_payloads(N, path):
    # Each bf16 buffer receives the binary32 mean rounded to nearest bf16,
    # ties to even, a NaN made quiet with its sign and leading payload kept;
    # the kernels narrow with gfx950's convert instruction, the oracle with an
    # integer rule on the bit pattern.  The elements cycle through the cases so
    # that every case falls in chunk heads, vector bodies and tails.
    ops, kinds = _bf16_rounding_cases(N)
    P = 3 * len(ops) + 11
    idx = np.arange(P) % len(ops)
    host = [np.ascontiguousarray(ops[idx, r]) for r in range(N)]
    d = _bf16_dev(host)
    if path in ("fused", "ring"):
        plan = api.rar_plan(N, P, api.BF16)
        api.rar_plan_set_algo(plan, api.FUSED if path == "fused" else api.RING)
        api.rar_allreduce_mean(plan, d, P)
    else:
        sizes = [P // 3, 5, P - P // 3 - 5]  # three tensors, buckets of 1000 elements
        b = api.rar_bucket_plan(sizes, api.BF16, 2 * 1000)
        cut = np.cumsum([0] + sizes)
        tensors = [[t[cut[i]:cut[i + 1]] for i in range(3)] for t in d]
        nb, mx = api.rar_bucket_count(b)
        if path == "bucket_tensors":
            api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.FUSED)
        else:
            bufs = [torch.empty(mx, dtype=torch.bfloat16, device=DEV) for _ in range(N)]
            api.rar_bucket_allreduce_mean(b, tensors, bufs, api.BALANCED, api.RING)
    # the binary32 means the same adds give on the device, from the binary32
    # fused pass over the widened inputs (same chunk table, same fold order)
    f32 = _to_dev([oracle.bf16_to_f32(h) for h in host])
    api.rar_allreduce_mean(api.rar_plan(N, P), f32, P)
    torch.cuda.synchronize()
    m32 = f32[0].cpu().numpy()
    assert np.all((m32[kinds[idx] == "tie"].view(np.uint32) & 0xFFFF) == 0x8000)
    assert np.all(np.isinf(m32[kinds[idx] == "overflow"]))
    # the narrowing itself, NaN payloads included: bit for bit with the oracle's
    # rule applied to the device's binary32 means
    want = oracle.f32_to_bf16(m32)
    ref = [h.copy() for h in host]
    oracle.ring_allreduce_bf16(ref, oracle.partition(N, P, api.BALANCED, 2))
    nan = kinds[idx] == "nan"
    assert np.all(np.isnan(oracle.bf16_to_f32(want[nan])))
    for n in range(N):
        got = _bits16(d[n])
        assert got.tobytes() == want.tobytes(), f"rank {n}: first diff {_first_diff(got, want)} ({kinds[idx][_first_diff(got, want)]})"
        # and the oracle end to end, NaN payloads included: with one NaN operand
        # both the device's and the host's binary32 adds return that NaN made quiet
        assert got.tobytes() == ref[n].tobytes(), f"rank {n}: first diff {_first_diff(got, ref[n])}"


@pytest.mark.parametrize("mode", [api.BALANCED, api.CEIL, api.ALIGN16])
@pytest.mark.parametrize("dt", [api.F32, api.BF16])
def test_buckets_with_tiny_and_empty_tensors(dt, mode):
    # empty tensors, one-element tensors and buckets smaller than N elements
    # (CEIL and ALIGN16 leave the last chunks of such buckets empty)
    N = 8
    numels = [0, 1, 0, 3, 1, 0, 17, 2, 1]
    es = 4 if dt == api.F32 else 2
    tdt = torch.float32 if dt == api.F32 else torch.bfloat16
    rng = np.random.default_rng(8)
    for bucket_elems in (1, 3, 5, 40):
        host = [[rng.integers(-9, 9, k).astype(np.float32) for k in numels] for _ in range(N)]
        tensors = [[torch.from_numpy(x.copy()).to(DEV).to(tdt) for x in rank] for rank in host]
        b = api.rar_bucket_plan(numels, dt, es * bucket_elems)
        for algo in (api.FUSED, api.RING):
            ts = [[t.clone() for t in rank] for rank in tensors]
            _, mx = api.rar_bucket_count(b)
            bufs = [torch.empty(max(mx, 1), dtype=tdt, device=DEV) for _ in range(N)]
            api.rar_bucket_allreduce_mean(b, ts, bufs, mode, algo)
            torch.cuda.synchronize()
            for t, k in enumerate(numels):
                S = sum(host[n][t].astype(np.float64) for n in range(N))
                expect = (S / N).astype(np.float32)  # integer inputs: every order is exact
                for n in (0, N - 1):
                    got = ts[n][t].float().cpu().numpy()
                    want = expect if dt == api.F32 else oracle.bf16_to_f32(oracle.f32_to_bf16(expect))
                    assert np.array_equal(got, want), (bucket_elems, algo, t, n)


# ---------------------------------------------------------------------------
# HIP graph capture: every call enqueues kernels only (no allocation, no
# synchronisation, no memset), so it can be captured and replayed
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["fused_sgd", "ring_sgd", "bf16_ring_sgd", "bucket_tensors", "bucket_tensors_ring"])
def test_graph_capture_replays_match_eager(path):
    N = 8
    if path.startswith("bucket_tensors"):
        specs = synth.transformer_tensors(1, d=64, h=256, V=900)
        numels = [s.numel for s in specs]
        b = api.rar_bucket_plan(numels, api.F32, 4 * 20_000)
        pristine = [[torch.randn(k, device=DEV) for k in numels] for _ in range(N)]
        live = [[t.clone() for t in rank] for rank in pristine]
        algo = api.RING if path.endswith("ring") else api.FUSED
        run = lambda: api.rar_bucket_allreduce_mean(b, live, None, api.BALANCED, algo)
        restore = lambda: [t.copy_(p) for rl, rp in zip(live, pristine) for t, p in zip(rl, rp)]
        state = lambda: torch.cat([t.reshape(-1) for rank in live for t in rank]).clone()
    else:
        P = 1_000_003
        dt = api.BF16 if path.startswith("bf16") else api.F32
        tdt = torch.bfloat16 if dt == api.BF16 else torch.float32
        plan = api.rar_plan(N, P, dt)
        api.rar_plan_set_algo(plan, api.FUSED if path == "fused_sgd" else api.RING)  # allocates now, not in capture
        pristine = [torch.randn(P, device=DEV).to(tdt) for _ in range(N)]
        w0 = torch.linspace(-0.05, 0.05, P, device=DEV)
        live = [t.clone() for t in pristine]
        w = w0.clone()
        run = lambda: api.rar_allreduce_sgd(plan, live, w, 0.01, P)
        restore = lambda: ([t.copy_(p) for t, p in zip(live, pristine)], w.copy_(w0))
        state = lambda: torch.cat([t.float() for t in live] + [w]).clone()
    # eager reference
    restore()
    run()
    torch.cuda.synchronize()
    eager = state()
    # capture (after a warm-up on a side stream, as torch requires)
    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        restore()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device=DEV).sum().item()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = state()
        assert torch.equal(got.view(torch.int32), eager.view(torch.int32)), f"{path}: replay {rep} differs"


def _random_bucket_cases(count=32, seed=77):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        N = int(rng.choice([2, 3, 4, 5, 8, 10, 16, 40]))
        dt = api.F32 if i % 3 else api.BF16
        algo = api.RING if i % 2 else api.FUSED
        mode = int(rng.integers(0, 3))
        n_t = int(rng.integers(1, 13))
        numels = [int(x) for x in rng.integers(0, 20_000, n_t)]
        numels[int(rng.integers(0, n_t))] += 1  # at least one element in all
        # from one element per bucket up, but at most ~200 buckets per case
        bucket_elems = max(int(rng.choice([1, 7, 64, 999, 4096, 30_001])), -(-sum(numels) // 200))
        views = bool(rng.integers(0, 2))
        cases.append((N, dt, algo, mode, tuple(numels), bucket_elems, views, int(rng.integers(0, 1 << 30))))
    return cases


@pytest.mark.parametrize("N,dt,algo,mode,numels,bucket_elems,views,seed", _random_bucket_cases())
def test_random_bucket_layouts_bit_exact(N, dt, algo, mode, numels, bucket_elems, views, seed):
    # random tensor lists (empty tensors included), bucket sizes from one
    # element up, every chunking, the fused and ring algorithms, tensors as
    # views of one arena per rank (adjacent pieces merge) or as separate
    # allocations: every element of every rank bit for bit against the
    # oracle's ring run bucket by bucket
    es = 4 if dt == api.F32 else 2
    tdt = torch.float32 if dt == api.F32 else torch.bfloat16
    rng = np.random.default_rng(seed)
    total = sum(numels)
    if dt == api.F32:
        host = [rng.standard_normal(total).astype(np.float32) for _ in range(N)]
    else:
        host = [oracle.f32_to_bf16(rng.standard_normal(total).astype(np.float32)) for _ in range(N)]
    cut = np.cumsum([0] + list(numels))
    keep, tensors = [], []
    for n in range(N):
        src = torch.from_numpy(host[n].view(np.int16) if dt == api.BF16 else host[n].copy()).to(DEV)
        src = src.view(tdt) if dt == api.BF16 else src
        if views:
            keep.append(src)
            tensors.append([src[cut[t]:cut[t + 1]] for t in range(len(numels))])
        else:
            tensors.append([src[cut[t]:cut[t + 1]].clone() for t in range(len(numels))])
    b = api.rar_bucket_plan(list(numels), dt, es * bucket_elems)
    _, mx = api.rar_bucket_count(b)
    bufs = [torch.empty(max(mx, 1), dtype=tdt, device=DEV) for _ in range(N)]
    api.rar_bucket_allreduce_mean(b, tensors, bufs, mode, algo)
    torch.cuda.synchronize()
    ref = [h.copy() for h in host]
    pos = 0
    for segs in oracle.bucket_layout(list(numels), es, es * bucket_elems):
        size = sum(sg[3] for sg in segs)
        part = [np.ascontiguousarray(r[pos:pos + size]) for r in ref]
        if dt == api.F32:
            oracle.ring_allreduce_f32(part, oracle.partition(N, size, mode, 4))
        else:
            oracle.ring_allreduce_bf16(part, oracle.partition(N, size, mode, 2))
        for n in range(N):
            ref[n][pos:pos + size] = part[n]
        pos += size
    for n in range(N):
        got = torch.cat([t.reshape(-1) for t in tensors[n]]) if total else torch.empty(0, dtype=tdt, device=DEV)
        got = got.cpu().numpy() if dt == api.F32 else _bits16(got)
        _assert_bits(got, ref[n], f"rank {n}")


# ---------------------------------------------------------------------------
# Buckets batched into shared launches: jobs of a full chunk (over 1 MiB per
# rank) and short ones (small tensors, bucket ends) go to separate batches
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,dt", [(2, api.F32), (4, api.F32), (8, api.F32), (10, api.F32), (16, api.F32),
                                  (40, api.F32), (4, api.BF16), (10, api.BF16), (40, api.BF16)])
def test_bucket_batches_mix_big_and_small_jobs(N, dt):
    es = 4 if dt == api.F32 else 2
    # chunk length just above the 1 MiB split (40 ranks: all jobs short, 8 per launch)
    c = (1 << 20) // es + 57_000 if N != 40 else 30_011
    B = N * c
    numels = [B + B // 2, 5, 2048, (7 * B) // 10 + 3, 17, B + 11, 1, 3000]
    total = sum(numels)
    rng = np.random.default_rng(1000 + N + es)
    if dt == api.F32:
        host = [rng.standard_normal(total, dtype=np.float32) * np.float32(1e-3) for _ in range(N)]
        tdt = torch.float32
    else:
        host = [synth.student_t3_bf16(total, 5000 + n, 1e-3, "cpu").view(torch.int16).numpy().view(np.uint16).copy()
                for n in range(N)]
        tdt = torch.bfloat16
    # expected values: each bucket packed and run through the oracle's literal ring
    layout = oracle.bucket_layout(numels, es, es * B)
    starts = np.concatenate([[0], np.cumsum(numels)])
    expect = [h.copy() for h in host]
    for segs in layout:
        size = sum(s[3] for s in segs)
        part = [np.concatenate([host[n][starts[t] + toff:starts[t] + toff + ln] for (t, toff, _, ln) in segs])
                for n in range(N)]
        if dt == api.F32:
            oracle.ring_allreduce_f32(part, oracle.partition(N, size))
        else:
            oracle.ring_allreduce_bf16(part, oracle.partition(N, size, oracle.BALANCED, 2))
        for n in range(N):
            for (t, toff, boff, ln) in segs:
                expect[n][starts[t] + toff:starts[t] + toff + ln] = part[n][boff:boff + ln]
    b = api.rar_bucket_plan(numels, dt, es * B)
    assert api.rar_bucket_count(b)[0] == len(layout)

    def upload():
        if dt == api.F32:
            return [torch.from_numpy(h.copy()).to(DEV) for h in host]
        return [torch.from_numpy(h.view(np.int16).copy()).to(DEV).view(torch.bfloat16) for h in host]

    for path in ("tensors", "arena"):
        arenas = upload()
        if path == "tensors":
            views = [[a[starts[t]:starts[t + 1]] for t in range(len(numels))] for a in arenas]
            api.rar_bucket_allreduce_mean(b, views, None, api.BALANCED, api.FUSED)
        else:
            api.rar_bucket_allreduce_arena(b, arenas, None, api.BALANCED, api.FUSED)
        torch.cuda.synchronize()
        for n in range(N):
            got = arenas[n].cpu()
            got = got.numpy() if dt == api.F32 else got.view(torch.int16).numpy().view(np.uint16)
            assert got.tobytes() == expect[n].tobytes(), \
                f"{path} rank {n}: first diff {_first_diff(got.view(np.uint32) if dt == api.F32 else got, expect[n].view(np.uint32) if dt == api.F32 else expect[n])}"
        del arenas


# ---------------------------------------------------------------------------
# Several host threads, each on its own stream, share one plan and one bucket
# handle (ctypes releases the GIL inside the library call)
# ---------------------------------------------------------------------------

def test_plan_and_buckets_shared_across_threads_and_streams():
    import threading
    N, T, ITERS = 8, 4, 6
    specs = synth.transformer_tensors(1, d=64, h=256, V=500)
    numels = [s.numel for s in specs]
    bucket_bytes = 4 * 9_000
    P = 100_003
    b = api.rar_bucket_plan(numels, api.F32, bucket_bytes)
    plan = api.rar_plan(N, P)
    work = []
    for th in range(T):
        rng = np.random.default_rng(700 + th)
        tens = [[rng.standard_normal(k).astype(np.float32) for k in numels] for _ in range(N)]
        flat = [rng.standard_normal(P).astype(np.float32) for _ in range(N)]
        w = rng.uniform(-0.05, 0.05, P).astype(np.float32)
        exp_t = [[x.copy() for x in rank] for rank in tens]
        oracle.bucketed_ring_f32(exp_t, bucket_bytes)
        exp_f = [x.copy() for x in flat]
        exp_w = w.copy()
        oracle.ring_allreduce_f32(exp_f, oracle.partition(N, P), exp_w, 0.01)
        work.append((tens, flat, w, exp_t, exp_f, exp_w))
    errors = []

    def run(th):
        try:
            tens, flat, w, exp_t, exp_f, exp_w = work[th]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for it in range(ITERS):
                    dt = [[torch.from_numpy(x).to(DEV, non_blocking=False) for x in rank] for rank in tens]
                    df = [torch.from_numpy(x).to(DEV) for x in flat]
                    dw = torch.from_numpy(w).to(DEV)
                    st.synchronize()
                    api.rar_bucket_allreduce_mean(b, dt, None, api.BALANCED, api.FUSED, stream=st)
                    api.rar_allreduce_sgd(plan, df, dw, 0.01, P, stream=st)
                    st.synchronize()
                    for n in (0, N - 1):
                        for t in range(len(numels)):
                            assert dt[n][t].cpu().numpy().tobytes() == exp_t[n][t].tobytes(), (th, it, n, t)
                        assert df[n].cpu().numpy().tobytes() == exp_f[n].tobytes(), (th, it, n)
                    assert dw.cpu().numpy().tobytes() == exp_w.tobytes(), (th, it)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(th,)) for th in range(T)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


# ---------------------------------------------------------------------------
# The C ABI from a plain C program (built by __graft_entry__.build())
# ---------------------------------------------------------------------------

def test_c_program_runs_the_abi_on_the_gpu():
    import subprocess
    exe = pathlib.Path(__file__).resolve().parent / "c_gpu_example.bin"
    assert exe.exists(), "tests/c_gpu_example.bin is not built: run __graft_entry__.build()"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-exact" in r.stdout


# ---------------------------------------------------------------------------
# Allocation failure is reported, not raised or crashed: a bf16 ring plan
# whose fp32 workspace cannot exist (2^40 floats = 4 TiB)
# ---------------------------------------------------------------------------

def test_workspace_allocation_failure_reports_enomem():
    plan = api.rar_plan(2, 1 << 40, api.BF16)
    with pytest.raises(api.RarError) as err:
        api.rar_plan_set_algo(plan, api.RING)
    assert err.value.status == api.ENOMEM
    # the plan is still usable with the algorithm it had, and the device is fine
    api.rar_plan_set_algo(plan, api.FUSED)
    x = torch.ones(1024, device=DEV)
    assert float(x.sum()) == 1024.0


# ---------------------------------------------------------------------------
# A seeded random sweep over shapes: rank counts with and without a
# compile-time kernel, ragged lengths, every chunking, both dtypes, every
# algorithm, mean and SGD, against the oracle bit for bit
# ---------------------------------------------------------------------------

def _random_cases(count=48, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        N = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 10, 13, 16, 17, 31, 40, 63, 64]))
        P = int(rng.integers(0, max(2, 3_000_000 // N)))
        if i % 5 == 0:
            P = int(rng.integers(0, 4 * N + 40))  # chunks of a few elements, empty ones
        dt = api.F32 if i % 3 else api.BF16
        mode = int(rng.integers(0, 3))
        algo = int(rng.integers(0, 3 if dt == api.F32 else 2))
        sgd = bool(rng.integers(0, 2))
        cases.append((N, P, dt, mode, algo, sgd))
    return cases


@pytest.mark.parametrize("N,P,dt,mode,algo,sgd", _random_cases())
def test_random_shapes_bit_exact(N, P, dt, mode, algo, sgd):
    lr = 0.05
    es = 4 if dt == api.F32 else 2
    if dt == api.F32:
        g = _host_f32(N, P, 31 * N + P % 1009)
        d = _to_dev(g)
    else:
        g = _host_bf16(N, P, 17 * N + P % 1009)
        d = _bf16_dev(g)
    w0 = np.random.default_rng(P % 7919).uniform(-0.05, 0.05, P).astype(np.float32)
    wd = torch.from_numpy(w0.copy()).to(DEV)
    plan = api.rar_plan(N, P, dt, mode)
    api.rar_plan_set_algo(plan, algo)
    if sgd:
        api.rar_allreduce_sgd(plan, d, wd, lr, P)
    else:
        api.rar_allreduce_mean(plan, d, P)
    torch.cuda.synchronize()
    ref = [x.copy() for x in g]
    wr = w0.copy()
    off = oracle.partition(N, P, mode, es)
    if dt == api.F32 and algo == api.NAIVE:
        oracle.naive_reduce_f32(ref, wr if sgd else None, lr)
    elif dt == api.F32:
        oracle.ring_allreduce_f32(ref, off, wr if sgd else None, lr)
    else:
        oracle.ring_allreduce_bf16(ref, off, wr if sgd else None, lr)
    for n in range(N):
        got = d[n].cpu().numpy() if dt == api.F32 else _bits16(d[n])
        if dt == api.F32:
            _assert_bits(got, ref[n], f"rank {n}")
        else:
            assert got.tobytes() == ref[n].tobytes(), f"rank {n}: first diff {_first_diff(got, ref[n])}"
    if sgd:
        _assert_bits(wd.cpu().numpy(), wr, "weights")


def test_graph_capture_arena_with_ready_events():
    """The overlap path captured whole: a producer stream forked from the
    capturing stream copies each bucket into the arenas and records the
    bucket's ready event; the reduction waits for them (one
    rar_bucket_allreduce_arena call).  Arenas start as NaN before every
    replay, so reducing a bucket before its copy would show."""
    N = 4
    specs = synth.transformer_tensors(1, d=64, h=256, V=900)
    numels = [s.numel for s in specs]
    total = sum(numels)
    b = api.rar_bucket_plan(numels, api.F32, 4 * 20_000)
    nb, _ = api.rar_bucket_count(b)
    infos = [api.rar_bucket_info(b, k) for k in range(nb)]
    pristine = [torch.randn(total, device=DEV) for _ in range(N)]
    arenas = [torch.empty(total, device=DEV) for _ in range(N)]
    events = [torch.cuda.Event() for _ in range(nb)]

    def step(main):
        prod = torch.cuda.Stream()
        prod.wait_stream(main)  # fork
        with torch.cuda.stream(prod):
            for k, (so, el, _) in enumerate(infos):
                for n in range(N):
                    arenas[n][so:so + el].copy_(pristine[n][so:so + el])
                events[k].record(prod)
        api.rar_bucket_allreduce_arena(b, arenas, events, stream=main)
        main.wait_stream(prod)  # join

    def poison():
        for a in arenas:
            a.fill_(float("nan"))

    poison()
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = torch.cat(arenas).clone()
    ref = [p.cpu().numpy().copy() for p in pristine]
    for k, (so, el, _) in enumerate(infos):
        part = [np.ascontiguousarray(r[so:so + el]) for r in ref]
        oracle.ring_allreduce_f32(part, oracle.partition(N, el))
        for n in range(N):
            ref[n][so:so + el] = part[n]
    _assert_bits(eager.cpu().numpy(), np.concatenate(ref), "eager")
    # warm-up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(arenas).view(torch.int32), eager.view(torch.int32)), f"replay {rep} differs"


# ---------------------------------------------------------------------------
# Rank buffers carved from one allocation at the library's recommended stride
# (the layout the benchmark uses): results do not depend on the layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("key,N,P", [(3, 10, 1_000_003), (5, 40, 400_003)])
@pytest.mark.parametrize("algo", [api.FUSED, api.RING])
def test_pooled_rank_layout_bit_exact(key, N, P, algo):
    wl = synth.WORKLOADS[key]
    dt = api.F32 if wl.dtype == "f32" else api.BF16
    stride = api.rar_rank_stride(P, dt)
    bufs = synth.rank_gradients_in_pool(wl, stride, DEV, P=P, N=N)
    assert all(b.data_ptr() - bufs[0].data_ptr() == n * stride for n, b in enumerate(bufs))
    w = synth.weights(wl, DEV, P=P)
    if dt == api.F32:
        ref = [b.cpu().numpy().copy() for b in bufs]
    else:
        ref = [b.view(torch.int16).cpu().numpy().view(np.uint16).copy() for b in bufs]
    wr = w.cpu().numpy().copy()
    plan = api.rar_plan(N, P, dt)
    api.rar_plan_set_algo(plan, algo)
    api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P)
    torch.cuda.synchronize()
    off = oracle.partition(N, P, api.BALANCED, 4 if dt == api.F32 else 2)
    if dt == api.F32:
        oracle.ring_allreduce_f32(ref, off, wr, wl.lr)
    else:
        oracle.ring_allreduce_bf16(ref, off, wr, wl.lr)
    for n in range(N):
        got = bufs[n].cpu().numpy() if dt == api.F32 else _bits16(bufs[n])
        assert got.tobytes() == ref[n].tobytes(), f"rank {n}"
    _assert_bits(w.cpu().numpy(), wr, "weights")


@pytest.mark.parametrize("key", [3, 5])
def test_rank_stride_tune_picks_a_fitting_candidate_and_stays_exact(key):
    """The measured layout advice returns one of the candidates that fit the
    pool, and the pass in that layout is bit-exact against the oracle."""
    MiB = 1 << 20
    wl = synth.WORKLOADS[key]
    dt = api.F32 if wl.dtype == "f32" else api.BF16
    tdt = torch.float32 if dt == api.F32 else torch.bfloat16
    es = 4 if dt == api.F32 else 2
    N, P, K = 6, 1_000_003, 4
    s0 = -(-P * es // (2 * MiB)) * 2 * MiB
    cands = [s0 + 2 * MiB * k for k in range(K)]
    assert cands == [api.rar_rank_stride_candidate(P, dt, k) for k in range(K)]
    pool = torch.zeros(synth.pool_elements(wl, cands[-1] + 2 * MiB, P, N), dtype=tdt, device=DEV)
    stride = api.rar_rank_stride_tune(N, P, dt, pool, candidates=K + 1)
    assert stride in cands + [cands[-1] + 2 * MiB]
    # the measurements behind a pick: with at most four candidates every one
    # is a finalist (24 timings); the smallest median wins unless the static
    # rule's stride is within a third of the median of the spreads
    pick, stats = api.rar_rank_stride_tune_stats(N, P, dt, pool, candidates=K)
    assert [c for c, _, _ in stats] == cands and pick in cands
    assert all(m > 0 and sp >= 0 for _, m, sp in stats)
    med = {c: m for c, m, _ in stats}
    best = min(cands, key=lambda c: (med[c], c))
    static = api.rar_rank_stride(P, dt)
    f = np.float32  # the library computes in binary32
    sp = sorted(f(s) for _, _, s in stats)
    typical = sp[K // 2] if K % 2 else f(f(sp[K // 2 - 1] + sp[K // 2]) * f(0.5))
    if static in med and static != best and f(f(med[static]) - f(med[best])) <= f(typical / f(3)):
        assert pick == static
    else:
        assert pick == best
    # more candidates asked for than fit: only those that fit are tried
    assert api.rar_rank_stride_tune(N, P, dt, pool, candidates=K + 20) in cands + [cands[-1] + 2 * MiB]
    # a pool that holds only the first candidate, and one element less
    exact = pool[:synth.pool_elements(wl, s0, P, N)]
    assert api.rar_rank_stride_tune(N, P, dt, exact, candidates=K) == s0
    with pytest.raises(api.RarError) as e:
        api.rar_rank_stride_tune(N, P, dt, exact[:-1], candidates=K)
    assert e.value.status == api.EINVAL
    # a pool holding 36 candidates: the tuner times exactly the library's candidate strides
    wide = torch.zeros(synth.pool_elements(wl, api.rar_rank_stride_candidate(P, dt, 35), P, N), dtype=tdt,
                       device=DEV)
    pick, stats = api.rar_rank_stride_tune_stats(N, P, dt, wide, candidates=64)
    assert [c for c, _, _ in stats] == [api.rar_rank_stride_candidate(P, dt, k) for k in range(36)]
    assert pick in [c for c, _, _ in stats]
    del wide
    torch.cuda.synchronize()
    bufs = synth.rank_gradients_in_pool(wl, stride, DEV, P=P, N=N, pool=pool)
    w = synth.weights(wl, DEV, P=P)
    if dt == api.F32:
        ref = [b.cpu().numpy().copy() for b in bufs]
    else:
        ref = [b.view(torch.int16).cpu().numpy().view(np.uint16).copy() for b in bufs]
    wr = w.cpu().numpy().copy()
    plan = api.rar_plan(N, P, dt)
    api.rar_allreduce_sgd(plan, bufs, w, wl.lr, P)
    torch.cuda.synchronize()
    off = oracle.partition(N, P, api.BALANCED, es)
    if dt == api.F32:
        oracle.ring_allreduce_f32(ref, off, wr, wl.lr)
    else:
        oracle.ring_allreduce_bf16(ref, off, wr, wl.lr)
    for n in range(N):
        got = bufs[n].cpu().numpy() if dt == api.F32 else _bits16(bufs[n])
        assert got.tobytes() == ref[n].tobytes(), f"rank {n}"
    _assert_bits(w.cpu().numpy(), wr, "weights")


@pytest.mark.parametrize("layout", ["contiguous", "gap_in_one_rank", "separate"])
def test_bucket_jobs_merge_only_across_contiguous_tensors(layout):
    """Pieces of consecutive tensors in one chunk become one job only where
    every rank's tensors are adjacent in memory; any layout reduces
    bit-exactly."""
    N = 8
    specs = synth.transformer_tensors(1, d=64, h=256, V=500)
    numels = [s.numel for s in specs]
    bucket_bytes = 4 * 20_000
    host = [[np.random.default_rng(900 + 100 * n + t).standard_normal(s.numel).astype(np.float32)
             for t, s in enumerate(specs)] for n in range(N)]
    ref = [[x.copy() for x in rank] for rank in host]
    oracle.bucketed_ring_f32(ref, bucket_bytes, api.BALANCED)
    b = api.rar_bucket_plan(numels, api.F32, bucket_bytes)
    tensors, keep = [], []
    for n in range(N):
        if layout == "separate":
            ts = [torch.from_numpy(x).to(DEV) for x in host[n]]
        else:
            # one flat arena; in rank 3 a 4-element gap after tensor 5
            gap = 4 if (layout == "gap_in_one_rank" and n == 3) else 0
            flat = torch.zeros(sum(numels) + gap, device=DEV)
            keep.append(flat)
            ts, pos = [], 0
            for t, k in enumerate(numels):
                ts.append(flat[pos:pos + k])
                ts[-1].copy_(torch.from_numpy(host[n][t]))
                pos += k + (gap if t == 5 else 0)
        tensors.append(ts)
    api.rar_bucket_allreduce_mean(b, tensors, None, api.BALANCED, api.FUSED)
    torch.cuda.synchronize()
    for n in range(N):
        for t in range(len(specs)):
            _assert_bits(tensors[n][t].cpu().numpy(), ref[n][t], f"{layout} rank {n} tensor {t}")


def _tuned_layout(wl, P, N, candidates=64):
    """The rank placement bench.py times: one pool, the stride the library
    measures fastest among `candidates` (the benchmark's 64)."""
    dt = api.F32 if wl.dtype == "f32" else api.BF16
    pool = torch.zeros(synth.pool_elements(wl, api.rar_rank_stride_candidate(P, dt, candidates - 1), P, N),
                       dtype=torch.float32 if dt == api.F32 else torch.bfloat16, device=DEV)
    stride = api.rar_rank_stride_tune(N, P, dt, pool, candidates)
    return stride, pool


@pytest.mark.parametrize("key", [3, 5])
def test_full_size_every_element(key):
    """The flat workloads at full size, in the layout and launch shape the
    benchmark times, through the fused pass and through the ring steps: every
    element of every rank, and the weights, bit-exact against the oracle run
    over the whole workload."""
    wl = synth.WORKLOADS[key]
    N, P = wl.N, wl.P
    bf16 = wl.dtype == "bf16"
    stride, pool = _tuned_layout(wl, P, N)
    g = synth.rank_gradients_in_pool(wl, stride, DEV, pool=pool)
    w = synth.weights(wl, DEV)
    ref = [_bits16(t).copy() if bf16 else t.cpu().numpy() for t in g]
    wr = w.cpu().numpy()
    off = oracle.partition(N, P, api.BALANCED, 2 if bf16 else 4)
    (oracle.ring_allreduce_bf16 if bf16 else oracle.ring_allreduce_f32)(ref, off, wr, wl.lr)
    for algo in (api.FUSED, api.RING):
        if algo == api.RING:  # fresh inputs in the same places
            g = synth.rank_gradients_in_pool(wl, stride, DEV, pool=pool)
            w = synth.weights(wl, DEV)
        plan = api.rar_plan(N, P, api.BF16 if bf16 else api.F32)
        api.rar_plan_set_algo(plan, algo)
        api.rar_allreduce_sgd(plan, g, w, wl.lr, P)
        torch.cuda.synchronize()
        for n in range(N):
            got = _bits16(g[n]) if bf16 else g[n].cpu().numpy()
            assert got.tobytes() == ref[n].tobytes(), \
                f"algo {algo} rank {n}: first difference at {_first_diff(got, ref[n])}"
        _assert_bits(w.cpu().numpy(), wr, f"algo {algo} weights")
        del plan


def test_full_size_transformer_buckets_every_element():
    """The 8-rank Transformer at full size (118 buckets of 25 MB, arenas at the
    benchmark's tuned stride), reduced by the fused pass straight from the
    tensor lists and as arena slices, and through the ring steps from the
    tensor lists (which lie end to end, so they take the arena launches and
    leave the bucket buffers unused): every element of every tensor
    bit-exact against the oracle's bucket-by-bucket literal ring."""
    wl = synth.WORKLOADS[4]
    stride, pool = _tuned_layout(wl, wl.P, wl.N)
    specs, ranks = synth.transformer_rank_tensors(wl, DEV, pool=pool, stride_bytes=stride)
    numels = [sp.numel for sp in specs]
    starts = np.concatenate([[0], np.cumsum(numels)])
    host = []
    for flat, _ in ranks:
        h = flat.cpu().numpy()
        host.append([h[starts[t]:starts[t + 1]] for t in range(len(numels))])
    oracle.bucketed_ring_f32(host, wl.bucket_bytes, api.BALANCED)
    want = [np.concatenate(h) for h in host]
    del host
    b = api.rar_bucket_plan(numels, api.F32, wl.bucket_bytes)
    _, mx = api.rar_bucket_count(b)
    for path in ("tensors", "arena", "ring"):
        if path != "tensors":  # fresh inputs in the same places
            specs, ranks = synth.transformer_rank_tensors(wl, DEV, pool=pool, stride_bytes=stride)
        if path == "tensors":
            api.rar_bucket_allreduce_mean(b, [ts for _, ts in ranks], None, api.BALANCED, api.FUSED)
        elif path == "arena":
            api.rar_bucket_allreduce_arena(b, [flat for flat, _ in ranks], None, api.BALANCED, api.FUSED)
        else:
            bufs = [torch.empty(mx, device=DEV) for _ in range(wl.N)]
            api.rar_bucket_allreduce_mean(b, [ts for _, ts in ranks], bufs, api.BALANCED, api.RING)
        torch.cuda.synchronize()
        for n, (flat, _) in enumerate(ranks):
            got = flat.cpu().numpy()
            assert got.tobytes() == want[n].tobytes(), \
                f"{path} rank {n}: first difference at {_first_diff(got, want[n])}"


def test_readme_python_example_runs():
    """The Python example in README.md runs as written and leaves every rank
    holding the same mean."""
    import pathlib
    import re
    text = (pathlib.Path(__file__).resolve().parents[1] / "README.md").read_text()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README has no python example"
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    grads, w = scope["grads"], scope["w"]
    assert len(grads) == scope["N"]
    for n in range(1, len(grads)):
        assert torch.equal(grads[n], grads[0]), f"rank {n}"
    assert torch.isfinite(w).all() and bool((w != 0).any())
