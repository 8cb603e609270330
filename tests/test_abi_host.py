"""The C ABI without a GPU: exports, host-side argument checks, and the host
tables (chunks, owners, traffic, buckets) against the oracle's independent
implementation.  No call here reaches a kernel launch: every execute call is
made with arguments the library must reject first, or with P == 0."""
import ctypes
import re
import pathlib

import pytest

import oracle
from ring_all_reduce_amd import api, synth
from ring_all_reduce_amd._lib import lib, SIGNATURES

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "rar.h"


def _declared():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rar_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 19
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(SIGNATURES) == names


def test_version_and_strerror():
    assert api.rar_version() >= 100
    for code in (api.OK, api.EINVAL, api.EMISMATCH, api.EALIGN, api.ENOMEM, api.EHIP, -99):
        assert isinstance(api.rar_strerror(code), str) and api.rar_strerror(code)


@pytest.mark.parametrize("N,P,dt,ch", [(0, 10, 0, 0), (65, 10, 0, 0), (4, -1, 0, 0), (4, 10, 2, 0),
                                       (4, 10, 0, 3), (-1, 0, 0, 0)])
def test_plan_rejects_bad_arguments(N, P, dt, ch):
    with pytest.raises(api.RarError) as e:
        api.rar_plan(N, P, dt, ch)
    assert e.value.status == api.EINVAL
    assert lib().rar_plan(4, 10, 0, 0, None) == api.EINVAL


@pytest.mark.parametrize("N,P", [(1, 0), (1, 7), (4, 1_000_003), (10, 11_700_000), (10, 300_000_000),
                                 (8, 781_250 * 8), (40, 100_000_000), (64, 63), (7, 3), (13, 1000)])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("dt", [0, 1])
def test_chunk_table_matches_oracle(N, P, mode, dt):
    eb = 4 if dt == 0 else 2
    plan = api.rar_plan(N, P, dt, mode)
    ref = oracle.partition(N, P, mode, eb)
    for c in range(N):
        off, ln, own = api.rar_plan_chunk(plan, c)
        assert (off, ln) == (ref[c], ref[c + 1] - ref[c])
        assert own == oracle.owner(c, N)
    with pytest.raises(api.RarError):
        api.rar_plan_chunk(plan, N)
    s_ref, r_ref = oracle.ring_traffic(N, ref)
    for n in range(N):
        assert api.rar_plan_traffic(plan, n) == (s_ref[n], r_ref[n])


def test_traffic_equals_page_formula_when_n_divides_p():
    N, P = 10, 300_000_000
    plan = api.rar_plan(N, P)
    for n in range(N):
        assert api.rar_plan_traffic(plan, n) == (2 * (N - 1) * P // N,) * 2


FAKE = 1 << 40  # never dereferenced: each call below must fail validation first


def _fake_bufs(N, P, es=4, gap=None):
    gap = gap if gap is not None else ((P * es + 4095) // 4096) * 4096 + 4096
    return [FAKE + i * gap for i in range(N)]


def test_execute_rejects_before_touching_the_device():
    N, P = 4, 1000
    plan = api.rar_plan(N, P)
    bufs = _fake_bufs(N, P)
    L = lib()
    assert L.rar_allreduce_mean(plan.handle, None, P, None) == api.EINVAL
    assert L.rar_allreduce_mean(None, api._ptr_array(bufs), P, None) == api.EINVAL
    assert L.rar_allreduce_mean(plan.handle, api._ptr_array(bufs), P + 1, None) == api.EMISMATCH
    assert L.rar_allreduce_mean(plan.handle, api._ptr_array(bufs[:3] + [0]), P, None) == api.EINVAL
    assert L.rar_allreduce_mean(plan.handle, api._ptr_array(bufs[:3] + [bufs[3] + 4]), P, None) == api.EALIGN
    assert L.rar_allreduce_mean(plan.handle, api._ptr_array(bufs[:3] + [bufs[0]]), P, None) == api.EINVAL
    overlap = bufs[:3] + [bufs[2] + 16 * ((P * 4) // 32)]
    assert L.rar_allreduce_mean(plan.handle, api._ptr_array(overlap), P, None) == api.EINVAL
    f = ctypes.c_float(0.1)
    assert L.rar_allreduce_sgd(plan.handle, api._ptr_array(bufs), None, f, P, None) == api.EINVAL
    assert L.rar_allreduce_sgd(plan.handle, api._ptr_array(bufs), bufs[1] + 64, f, P, None) == api.EINVAL
    assert L.rar_allreduce_sgd(plan.handle, api._ptr_array(bufs), FAKE - 8, f, P, None) == api.EALIGN
    assert L.rar_reduce_scatter_sgd_allgather(plan.handle, api._ptr_array(bufs), None, f, P, None) == api.EINVAL
    wdup = api._ptr_array([FAKE + (1 << 36)] * N)
    assert L.rar_reduce_scatter_sgd_allgather(plan.handle, api._ptr_array(bufs), wdup, f, P, None) == api.EINVAL


def test_binding_checks_tensor_dtype_and_size_before_the_call():
    # The library sees only addresses; the binding checks a tensor's element
    # type and length against the plan before handing its address over, so a
    # bf16 tensor for a binary32 plan, or a short buffer, cannot make the
    # kernels run past an allocation.  CPU tensors: the checks come first.
    import torch
    N, P = 3, 10
    f32 = [torch.zeros(P) for _ in range(N)]
    plan = api.rar_plan(N, P)
    bplan = api.rar_plan(N, P, api.BF16)
    w = torch.zeros(P)
    bad = {
        "bf16 buffer for a binary32 plan": lambda: api.rar_allreduce_mean(plan, f32[:2] + [f32[2].bfloat16()], P),
        "binary32 buffer for a bf16 plan": lambda: api.rar_allreduce_mean(bplan, f32, P),
        "short buffer": lambda: api.rar_allreduce_mean(plan, f32[:2] + [torch.zeros(P - 1)], P),
        "short w": lambda: api.rar_allreduce_sgd(plan, f32, torch.zeros(P - 1), 0.1, P),
        "float64 w": lambda: api.rar_allreduce_sgd(plan, f32, torch.zeros(P, dtype=torch.float64), 0.1, P),
        "bf16 w": lambda: api.rar_allreduce_sgd(bplan, [t.bfloat16() for t in f32], w.bfloat16(), 0.1, P),
        "short w replica": lambda: api.rar_reduce_scatter_sgd_allgather(plan, f32, [w, w.clone(), w[:5]], 0.1, P),
    }
    for what, call in bad.items():
        with pytest.raises(ValueError):
            call()
    numels = [7, 0, 13]
    b = api.rar_bucket_plan(numels, api.F32, 4 * 8)
    nb, mx = api.rar_bucket_count(b)
    ok = [[torch.zeros(n) for n in numels] for _ in range(N)]
    short = [[torch.zeros(n) for n in numels] for _ in range(N - 1)] + [[torch.zeros(7), torch.zeros(0),
                                                                           torch.zeros(12)]]
    wrong = [[torch.zeros(n) for n in numels] for _ in range(N - 1)] + [[torch.zeros(n, dtype=torch.bfloat16)
                                                                           for n in numels]]
    bucket_bad = {
        "short tensor": lambda: api.rar_bucket_allreduce_mean(b, short, None),
        "bf16 tensor in a binary32 bucket plan": lambda: api.rar_bucket_allreduce_mean(b, wrong, None),
        "short bucket buffer": lambda: api.rar_bucket_allreduce_mean(b, ok, [torch.zeros(mx)] * 2 + [torch.zeros(mx - 1)],
                                                                     algo=api.RING),
        "short pack buffer": lambda: api.rar_bucket_pack(b, 0, ok, [torch.zeros(8)] * 2 + [torch.zeros(7)]),
        "short unpack buffer": lambda: api.rar_bucket_unpack(b, 0, [torch.zeros(8)] * 2 + [torch.zeros(7)], ok),
        "short arena": lambda: api.rar_bucket_allreduce_arena(b, [torch.zeros(20)] * 2 + [torch.zeros(19)]),
        "bf16 arena": lambda: api.rar_bucket_allreduce_arena(b, [torch.zeros(20, dtype=torch.bfloat16)] * 3),
    }
    for what, call in bucket_bad.items():
        with pytest.raises(ValueError):
            call()
    # what passes the checks reaches the next one: CPU tensors are not device memory
    for call in (lambda: api.rar_allreduce_sgd(plan, f32, w, 0.1, P),
                 lambda: api.rar_bucket_allreduce_arena(b, [torch.zeros(20)] * 3)):
        with pytest.raises(ValueError, match="on the GPU"):
            call()
    # a P that differs from the plan's is still the library's RAR_EMISMATCH
    with pytest.raises(api.RarError):
        api.rar_allreduce_mean(plan, [0x10000000, 0x20000000, 0x30000000], P + 1)


def test_noalloc_ring_rejects_before_touching_the_device():
    # checks of rar_allreduce_mean / _sgd, then the static workspace's limit,
    # all before the first HIP call
    L, f = lib(), ctypes.c_float(0.1)
    big = api.STATIC_WS_ELEMS + 1
    bplan = api.rar_plan(4, big, api.BF16)
    bufs = api._ptr_array(_fake_bufs(4, big, 2))
    assert L.rar_allreduce_ring_noalloc(bplan.handle, bufs, None, f, big, None) == api.ETOOLARGE
    assert api.rar_strerror(api.ETOOLARGE) == "element count exceeds the static workspace"
    assert L.rar_allreduce_ring_noalloc(bplan.handle, bufs, None, f, big - 1, None) == api.EMISMATCH
    assert L.rar_allreduce_ring_noalloc(bplan.handle, None, None, f, big, None) == api.EINVAL
    wbad = _fake_bufs(4, big, 2)[1] + 64  # inside a rank buffer
    assert L.rar_allreduce_ring_noalloc(bplan.handle, bufs, wbad, f, big, None) == api.EINVAL
    plan = api.rar_plan(4, 1000)
    fb = _fake_bufs(4, 1000)
    assert L.rar_allreduce_ring_noalloc(plan.handle, api._ptr_array(fb[:3] + [fb[3] + 4]), None, f, 1000,
                                        None) == api.EALIGN
    api.rar_allreduce_ring_noalloc(api.rar_plan(3, 0, api.BF16), [0, 0, 0], None, 0.1, 0, stream=0)  # no-op


def test_zero_elements_is_a_no_op():
    plan = api.rar_plan(3, 0)
    api.rar_allreduce_mean(plan, [0, 0, 0], 0, stream=0)
    api.rar_allreduce_sgd(plan, [0, 0, 0], 0, 0.1, 0, stream=0)


def test_set_algo_and_grid_checks():
    plan = api.rar_plan(4, 100, api.BF16)
    with pytest.raises(api.RarError):
        api.rar_plan_set_algo(plan, api.NAIVE)
    with pytest.raises(api.RarError):
        api.rar_plan_set_algo(plan, 7)
    with pytest.raises(api.RarError):
        api.rar_plan_set_grid(plan, -1)
    f32 = api.rar_plan(4, 100)
    for a in (api.FUSED, api.RING, api.NAIVE):
        api.rar_plan_set_algo(f32, a)  # no workspace for binary32: no device call
    api.rar_plan_set_grid(f32, 17)


def test_bucket_layout_matches_oracle():
    specs = synth.transformer_tensors(12)
    numels = [s.numel for s in specs]
    b = api.rar_bucket_plan(numels, api.F32, 25_000_000)
    ref = oracle.bucket_layout(numels, 4, 25_000_000)
    nb, mx = api.rar_bucket_count(b)
    assert nb == len(ref) == 118 and mx == 6_250_000
    pos = 0
    for k, segs in enumerate(ref):
        so, el, ns = api.rar_bucket_info(b, k)
        assert so == pos and el == sum(s[3] for s in segs) and ns == len(segs)
        for j, seg in enumerate(segs):
            assert api.rar_bucket_segment(b, k, j) == tuple(seg)
        pos += el
    assert api.rar_bucket_info(b, 117)[1] == 4_121_264


@pytest.mark.parametrize("numels,bb,dt", [([5, 0, 7, 100, 1], 8, 0), ([3] * 10, 4, 1), ([], 16, 0),
                                          ([1000], 4000, 0), ([1000], 4004, 0)])
def test_bucket_layout_small_cases(numels, bb, dt):
    b = api.rar_bucket_plan(numels, dt, bb)
    ref = oracle.bucket_layout(numels, 4 if dt == 0 else 2, bb)
    assert api.rar_bucket_count(b)[0] == len(ref)
    for k, segs in enumerate(ref):
        assert [api.rar_bucket_segment(b, k, j) for j in range(len(segs))] == [tuple(s) for s in segs]


def test_bucket_plan_rejects_bad_arguments():
    for args in (([1, -1], 0, 16), ([1], 0, 3), ([1], 5, 16), ([1], 1, 1)):
        with pytest.raises(api.RarError):
            api.rar_bucket_plan(*args)


def test_bucket_arena_checks_alignment_and_arguments():
    L = lib()
    b = api.rar_bucket_plan([10, 7, 30], api.F32, 12)  # 3-element buckets start at 12-byte multiples
    ar = api._ptr_array([FAKE, FAKE + (1 << 20)])
    assert L.rar_bucket_allreduce_arena(b.handle, 2, 0, 0, ar, None, None) == api.EALIGN
    b16 = api.rar_bucket_plan([10, 7, 30], api.F32, 16)
    assert L.rar_bucket_allreduce_arena(b16.handle, 2, 0, 0, api._ptr_array([FAKE + 4, FAKE + (1 << 20)]),
                                        None, None) == api.EALIGN
    assert L.rar_bucket_allreduce_arena(b16.handle, 2, 0, 0, api._ptr_array([FAKE, 0]), None, None) == api.EINVAL
    assert L.rar_bucket_allreduce_arena(b16.handle, 0, 0, 0, ar, None, None) == api.EINVAL
    assert L.rar_bucket_allreduce_arena(None, 2, 0, 0, ar, None, None) == api.EINVAL


def test_header_is_plain_c_and_links(tmp_path):
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    from ring_all_reduce_amd._lib import LIB_PATH
    exe = tmp_path / "c_abi_check"
    src = pathlib.Path(__file__).resolve().parent / "c_abi_check.c"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{ROOT / 'include'}",
                    str(src), str(LIB_PATH), f"-Wl,-rpath,{LIB_PATH.parent}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout


def test_bucket_tensors_must_not_overlap_across_ranks():
    L = lib()
    b = api.rar_bucket_plan([100, 50], api.F32, 4 * 64)
    # rank-major pointers: rank 0 (t0, t1), rank 1 (t0, t1); rank 1's tensor 0 is rank 0's tensor 0
    same = api._ptr_array([FAKE, FAKE + 4096, FAKE, FAKE + 8192])
    bufs = api._ptr_array([FAKE + (1 << 30), FAKE + (1 << 30) + 4096])
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 0, same, bufs, None) == api.EINVAL
    assert L.rar_bucket_pack(b.handle, 0, 2, same, bufs, None) == api.EINVAL


def test_bucket_buffers_must_not_overlap_each_other_or_the_tensors():
    """Only layouts that must fail validation (FAKE is never dereferenced);
    the tight layouts that pass are exercised on the GPU."""
    L = lib()
    b = api.rar_bucket_plan([100, 50], api.F32, 4 * 64)  # buckets of 64, 64, 22 elements
    tensors = api._ptr_array([FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288])
    far = FAKE + (1 << 30)
    # bucket 0 needs 256 bytes per buffer: buffers 240 bytes apart overlap
    close = api._ptr_array([far, far + 240])
    assert L.rar_bucket_pack(b.handle, 0, 2, tensors, close, None) == api.EINVAL
    assert L.rar_bucket_unpack(b.handle, 0, 2, close, tensors, None) == api.EINVAL
    # bucket 2 holds 22 elements (88 bytes): 80 bytes apart overlap
    assert L.rar_bucket_pack(b.handle, 2, 2, tensors, api._ptr_array([far, far + 80]), None) == api.EINVAL
    # a bucket buffer over rank 1's tensor 0 (bucket 0 reads FAKE+8192 .. +256 of rank 1)
    over = api._ptr_array([far, FAKE + 8192 + 128])
    assert L.rar_bucket_pack(b.handle, 0, 2, tensors, over, None) == api.EINVAL
    assert L.rar_bucket_unpack(b.handle, 0, 2, over, tensors, None) == api.EINVAL
    # ... or starting before rank 0's tensor 0 and running into it
    assert L.rar_bucket_pack(b.handle, 0, 2, tensors, api._ptr_array([FAKE - 128, far]), None) == api.EINVAL
    # the packing path of the bucketed all-reduce checks the buffers too
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 1, tensors, over, None) == api.EINVAL
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 1, tensors, close, None) == api.EINVAL


def test_bucket_tensors_must_not_overlap_across_tensors_or_buckets():
    """Jobs of consecutive buckets share a launch, so the direct path rejects
    any two tensors (of any ranks, in any buckets) that share memory."""
    L = lib()
    # 64-element buckets: tensor 0 (100) fills bucket 0 and part of bucket 1, tensor 1 (50) the rest
    b = api.rar_bucket_plan([100, 50], api.F32, 4 * 64)
    assert api.rar_bucket_count(b)[0] == 3
    # rank 0's tensor 1 starts inside rank 0's tensor 0 (different buckets)
    alias = api._ptr_array([FAKE, FAKE + 200, FAKE + 4096, FAKE + 8192])
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 0, alias, None, None) == api.EINVAL
    # rank 1's tensor 1 overlaps rank 0's tensor 0's last element
    alias = api._ptr_array([FAKE, FAKE + 4096, FAKE + 8192, FAKE + 396])
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 0, alias, None, None) == api.EINVAL
    # a null pointer for a non-empty tensor
    alias = api._ptr_array([FAKE, FAKE + 4096, FAKE + 8192, 0])
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 0, alias, None, None) == api.EINVAL


def test_bucket_arenas_must_not_overlap():
    L = lib()
    b = api.rar_bucket_plan([100, 50], api.F32, 4 * 64)  # 150 elements = 600 bytes per arena
    assert L.rar_bucket_allreduce_arena(b.handle, 2, 0, 0, api._ptr_array([FAKE, FAKE + 592]),
                                        None, None) == api.EINVAL
    assert L.rar_bucket_allreduce_arena(b.handle, 2, 0, 0, api._ptr_array([FAKE, FAKE]), None, None) == api.EINVAL


def test_bucket_plan_rejects_layouts_beyond_int_indices():
    L = lib()
    out = ctypes.c_void_p()
    # 2^40 one-element buckets: more than an int can index
    arr = (ctypes.c_int64 * 1)(1 << 40)
    assert L.rar_bucket_plan(1, arr, api.F32, 4, ctypes.byref(out)) == api.EINVAL
    # element counts whose sum overflows int64
    arr = (ctypes.c_int64 * 2)((1 << 63) - 1, 1)
    assert L.rar_bucket_plan(2, arr, api.F32, 1 << 30, ctypes.byref(out)) == api.EINVAL


def test_bucket_calls_validate_arguments_even_without_buckets():
    L = lib()
    b = api.rar_bucket_plan([], api.F32)
    assert api.rar_bucket_count(b)[0] == 0
    empty = api._ptr_array([])
    for N, chunking, algo in ((0, 0, 0), (65, 0, 0), (2, 7, 0), (2, 0, 9)):
        assert L.rar_bucket_allreduce_mean(b.handle, N, chunking, algo, empty, None, None) == api.EINVAL
        assert L.rar_bucket_allreduce_arena(b.handle, N, chunking, algo, api._ptr_array([FAKE] * max(N, 1)),
                                            None, None) == api.EINVAL
    assert L.rar_bucket_allreduce_mean(b.handle, 2, 0, 0, empty, None, None) == api.OK


def test_null_tensor_pointers_are_rejected_before_any_device_work():
    """Tensor lists with null pointers, for every algorithm: the check of
    whether the lists lie end to end (made before validation) treats them as
    no arena, and validation rejects the call.  Run on the CPU, so nothing may
    reach a launch."""
    L = lib()
    for dt in (api.F32, api.BF16):
        b = api.rar_bucket_plan([100, 0, 60, 4], dt, 64)
        N = 3
        null = api._ptr_array([None] * (N * 4))
        # first rank's tensors end to end, the others null
        es = 4 if dt == api.F32 else 2
        part = api._ptr_array([FAKE, FAKE + 100 * es, FAKE + 100 * es, FAKE + 160 * es] + [None] * (2 * 4))
        for algo in (api.FUSED, api.RING, api.NAIVE):
            if dt == api.BF16 and algo == api.NAIVE:
                continue
            for tensors in (null, part):
                assert L.rar_bucket_allreduce_mean(b.handle, N, api.BALANCED, algo, tensors, None, None) == api.EINVAL


def test_binding_rejects_ragged_tensor_lists_and_short_event_lists():
    b = api.rar_bucket_plan([10, 20], api.F32, 4 * 16)
    ragged = [[FAKE, FAKE + 4096], [FAKE + 8192]]
    with pytest.raises(ValueError):
        api.rar_bucket_allreduce_mean(b, ragged)
    with pytest.raises(ValueError):
        api.rar_bucket_pack(b, 0, ragged, [FAKE + (1 << 30), FAKE + (1 << 31)])
    with pytest.raises(ValueError):
        api.rar_bucket_allreduce_arena(b, [FAKE, FAKE + (1 << 20)], ready_events=[None])


def test_binding_rejects_pointer_lists_of_the_wrong_length():
    plan = api.rar_plan(4, 100)
    for bad in ([FAKE] * 3, [FAKE] * 5):
        with pytest.raises(ValueError):
            api.rar_allreduce_mean(plan, bad, 100)
        with pytest.raises(ValueError):
            api.rar_allreduce_sgd(plan, bad, FAKE + (1 << 30), 0.1, 100)
    with pytest.raises(ValueError):
        api.rar_reduce_scatter_sgd_allgather(plan, [FAKE + (i << 20) for i in range(4)], [FAKE + (1 << 30)], 0.1, 100)


# ---------------------------------------------------------------------------
# Property tests of the host tables against the oracle over random shapes
# ---------------------------------------------------------------------------

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=300, deadline=None)
@given(N=st.integers(1, 64), P=st.integers(0, 10 ** 7), mode=st.sampled_from([api.BALANCED, api.CEIL, api.ALIGN16]),
       dt=st.sampled_from([api.F32, api.BF16]))
def test_chunk_table_owner_and_traffic_match_the_oracle(N, P, mode, dt):
    es = 4 if dt == api.F32 else 2
    plan = api.rar_plan(N, P, dt, mode)
    off = oracle.partition(N, P, mode, es)
    sent_o, recv_o = oracle.ring_traffic(N, off)
    for c in range(N):
        o, ln, own = api.rar_plan_chunk(plan, c)
        assert (o, ln) == (int(off[c]), int(off[c + 1] - off[c]))
        assert own == oracle.owner(c, N)
    for n in range(N):
        assert api.rar_plan_traffic(plan, n) == (int(sent_o[n]), int(recv_o[n]))


@settings(max_examples=200, deadline=None)
@given(numels=st.lists(st.integers(0, 5000), min_size=0, max_size=40),
       bucket_elems=st.integers(1, 3000), dt=st.sampled_from([api.F32, api.BF16]))
def test_bucket_layout_matches_the_oracle_on_random_lists(numels, bucket_elems, dt):
    es = 4 if dt == api.F32 else 2
    b = api.rar_bucket_plan(numels, dt, es * bucket_elems)
    layout = oracle.bucket_layout(numels, es, es * bucket_elems)
    nb, mx = api.rar_bucket_count(b)
    assert nb == len(layout)
    assert mx == max((sum(sg[3] for sg in segs) for segs in layout), default=0)
    start = 0
    for k, segs in enumerate(layout):
        so, el, ns = api.rar_bucket_info(b, k)
        assert (so, el, ns) == (start, sum(sg[3] for sg in segs), len(segs))
        for j, sg in enumerate(segs):
            assert api.rar_bucket_segment(b, k, j) == tuple(int(x) for x in sg)
        start += el


def test_rank_stride_is_two_mib_modulo_four_and_covers_the_buffer():
    MiB = 1 << 20
    for P, dt in ((0, api.F32), (1, api.F32), (300_000_000, api.F32), (100_000_000, api.BF16),
                  (524_288, api.F32), (524_289, api.F32), (1_572_864, api.F32), (1_572_865, api.F32)):
        es = 4 if dt == api.F32 else 2
        s = api.rar_rank_stride(P, dt)
        assert s % (4 * MiB) == 2 * MiB and s >= P * es
        assert s - 4 * MiB < max(P * es, 2 * MiB)  # the smallest such stride
    assert api.rar_rank_stride(300_000_000) == 1146 * MiB
    L = lib()
    out = ctypes.c_int64()
    assert L.rar_rank_stride(-1, 0, ctypes.byref(out)) == api.EINVAL
    assert L.rar_rank_stride(10, 7, ctypes.byref(out)) == api.EINVAL
    assert L.rar_rank_stride(10, 0, None) == api.EINVAL
    assert L.rar_rank_stride((1 << 62), 0, ctypes.byref(out)) == api.EINVAL


def test_rank_stride_candidates():
    """The tuner's candidate strides: 32 at 2 MiB steps from the smallest
    multiple of 2 MiB that holds a rank, then 32 multiples of 8 MiB from the
    first one at least 64 MiB past it; rar_rank_stride's stride among the
    first two."""
    MiB = 1 << 20
    for P, dt in ((300_000_000, api.F32), (100_000_000, api.BF16), (11_700_000, api.F32), (1, api.F32), (0, api.BF16),
                  (735_371_264, api.F32)):
        es = 4 if dt == api.F32 else 2
        s0 = max(2 * MiB, -(-P * es // (2 * MiB)) * 2 * MiB)
        c = [api.rar_rank_stride_candidate(P, dt, k) for k in range(api.MAX_STRIDE_CANDIDATES)]
        assert c[:32] == [s0 + 2 * MiB * k for k in range(32)]
        c0 = -(-(s0 + 64 * MiB) // (8 * MiB)) * 8 * MiB
        assert c[32:] == [c0 + 8 * MiB * k for k in range(32)]
        assert all(a < b for a, b in zip(c, c[1:])) and c[0] >= P * es
        assert api.rar_rank_stride(P, dt) in c[:2]
    for args in ((-1, api.F32, 0), (10, 7, 0), (10, api.F32, -1), (10, api.F32, api.MAX_STRIDE_CANDIDATES)):
        with pytest.raises(api.RarError):
            api.rar_rank_stride_candidate(*args)
    assert lib().rar_rank_stride_candidate(10, api.F32, 0, None) == api.EINVAL


def test_rank_stride_tune_validates_before_any_device_work():
    """Only calls that must return before device work (FAKE is never
    dereferenced); the measurement itself runs on the GPU."""
    MiB = 1 << 20
    L = lib()
    out = ctypes.c_int64()
    big = 1 << 34
    # nothing to place: the smallest candidate, no pool needed
    assert L.rar_rank_stride_tune(1, 300_000_000, api.F32, None, 0, 4, None, ctypes.byref(out)) == api.OK
    assert out.value == 1146 * MiB
    assert L.rar_rank_stride_tune(8, 0, api.BF16, None, 0, 4, None, ctypes.byref(out)) == api.OK
    assert out.value == 2 * MiB
    assert L.rar_rank_stride_tune(1, 100_000_000, api.BF16, None, 0, 1, None, ctypes.byref(out)) == api.OK
    assert out.value == 192 * MiB  # 200 MB rounds up to 191 MiB, then to a multiple of 2 MiB
    bad = [
        (4, 1000, api.F32, None, big, 4),                          # no pool
        (4, 1000, api.F32, FAKE, 6 * MiB, 4),                      # 3 * 2 MiB + 4000 bytes do not fit
        (4, 1000, api.F32, FAKE, big, 0),                          # no candidates
        (4, 1000, api.F32, FAKE, big, 65),                         # beyond RAR_MAX_STRIDE_CANDIDATES
        (0, 1000, api.F32, FAKE, big, 4), (65, 1000, api.F32, FAKE, big, 4),
        (4, 1000, 7, FAKE, big, 4), (4, -1, api.F32, FAKE, big, 4),
        (4, 1 << 62, api.F32, FAKE, big, 4),
    ]
    for args in bad:
        assert L.rar_rank_stride_tune(*args, None, ctypes.byref(out)) == api.EINVAL, args
    assert L.rar_rank_stride_tune(4, 1000, api.F32, FAKE + 8, big, 4, None, ctypes.byref(out)) == api.EALIGN
    assert L.rar_rank_stride_tune(4, 1000, api.F32, FAKE, big, 4, None, None) == api.EINVAL
    with pytest.raises(TypeError):
        api.rar_rank_stride_tune(4, 1000, api.F32, FAKE)
