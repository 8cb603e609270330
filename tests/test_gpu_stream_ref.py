"""The benchmark's reference stream kernels (libstream_ref.so) move what they
claim: the in-place movers leave every buffer as it was, the copy copies, the
write-only kernel writes every vector of every stream and nothing past them,
the read-only kernel writes nothing.  They are not part of the all-reduce;
bench.py times them as the ceiling of the fused pass's access pattern, and
these checks make sure those rows moved the bytes they are credited with."""
import ctypes
import pathlib

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
LIB = ROOT / "ring_all_reduce_amd" / "libstream_ref.so"
LANES = 256


def _lib():
    if not LIB.exists():
        pytest.fail(f"{LIB} is not built; run `python -m ring_all_reduce_amd.build`")
    L = ctypes.CDLL(str(LIB))
    L.sref_run.restype = ctypes.c_int
    L.sref_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                           ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def _arr(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def test_reference_kernels_reject_bad_shapes_without_launching():
    L = _lib()
    a, b = 1 << 20, 1 << 21
    ranks10 = _arr([a + (i << 16) for i in range(10)])
    w = 1 << 24
    # unknown mode, no ranks, negative size
    assert L.sref_run(5, 10, ranks10, w, 1, 64, 4, None, None) == -1
    assert L.sref_run(0, 0, ranks10, w, 1, 64, 4, None, None) == -1
    assert L.sref_run(0, 10, ranks10, w, 1, -1, 4, None, None) == -1
    # a shape without a compiled kernel, a weight stream without its vector count
    assert L.sref_run(0, 10, ranks10, w, 1, 64, 3, None, None) == -1
    assert L.sref_run(0, 10, ranks10, None, 1, 64, 4, None, None) == -1
    # misaligned rank pointer, read-only without a sink
    assert L.sref_run(0, 10, _arr([a + 8] + [a + (i << 16) for i in range(1, 10)]), w, 1, 64, 4, None, None) == -1
    assert L.sref_run(2, 10, ranks10, w, 1, 64, 4, None, None) == -1
    # the table mover exists for 10 binary32 ranks with weights only
    assert L.sref_run(4, 40, _arr([a + (i << 16) for i in range(40)]), w, 2, 64, 4, None, None) == -1
    assert L.sref_run(4, 10, ranks10, w, 1, 64, 1, None, None) == -1
    # the copy needs two ranks that do not overlap
    assert L.sref_run(3, 2, _arr([a, a + 512]), None, 0, 64, 1, None, None) == -1
    assert L.sref_run(3, 3, _arr([a, b, b + (1 << 16)]), None, 0, 64, 1, None, None) == -1
    # zero vectors: nothing to launch
    assert L.sref_run(0, 10, ranks10, w, 1, 0, 4, None, None) == 0


SHAPES = [  # (mode, ranks, groups, w vectors per lane)
    (0, 10, 4, 1), (0, 10, 1, 1), (0, 40, 4, 2), (0, 8, 4, 0), (0, 1, 1, 0), (4, 10, 4, 1),
    (1, 10, 4, 1), (1, 10, 1, 1), (1, 40, 4, 2), (1, 1, 1, 0), (2, 10, 4, 1), (2, 40, 4, 2), (2, 1, 1, 0),
    (3, 2, 1, 0),
]


@pytest.mark.gpu
@pytest.mark.parametrize("vecs", [1, 255, 1000, 3 * LANES])
@pytest.mark.parametrize("mode,n,groups,wv", SHAPES)
def test_reference_kernels_move_what_they_claim(mode, n, groups, wv, vecs):
    import torch
    L = _lib()
    dev = torch.device("cuda:0")
    pad = 64  # vectors past the end of every stream, which must stay untouched
    gen = torch.Generator(device="cpu").manual_seed(1000 * mode + 10 * n + groups + vecs)
    ranks = [torch.randint(-2**31, 2**31 - 1, ((vecs + pad) * 4,), generator=gen, dtype=torch.int32).to(dev)
             for _ in range(n)]
    w = (torch.randint(-2**31, 2**31 - 1, ((wv * vecs + pad) * 4,), generator=gen, dtype=torch.int32).to(dev)
         if wv else None)
    sink = torch.zeros(LANES * 4, dtype=torch.int32, device=dev)
    before = [r.clone() for r in ranks]
    w_before = w.clone() if w is not None else None
    stream = torch.cuda.current_stream(dev)
    print(f"sref_run mode={mode} ranks={n} groups={groups} w_vpl={wv} vecs={vecs}", flush=True)
    rc = L.sref_run(mode, n, _arr([r.data_ptr() for r in ranks]), w.data_ptr() if w is not None else None, wv,
                    vecs, groups, sink.data_ptr(), stream.cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    body = vecs * 4
    for r, b in zip(ranks, before):
        assert torch.equal(r[body:], b[body:]), "a stream was written past its end"
    if w is not None:
        assert torch.equal(w[wv * body:], w_before[wv * body:]), "the weight stream was written past its end"
    if mode in (0, 2, 4):  # moved in place unchanged, or only read
        for r, b in zip(ranks, before):
            assert torch.equal(r, b)
        if w is not None:
            assert torch.equal(w, w_before)
        assert not sink.any()
    elif mode == 3:
        assert torch.equal(ranks[1][:body], before[0][:body])
        assert torch.equal(ranks[0], before[0])
    else:  # write only: vector v of group g's streams holds (v mod 256, g, 0, 0)
        per = -(-n // groups)
        lane = torch.arange(vecs, device=dev, dtype=torch.int32) % LANES
        for k, r in enumerate(ranks):
            v = r[:body].view(vecs, 4)
            assert torch.equal(v[:, 0], lane) and (v[:, 1] == k // per).all() and not v[:, 2:].any()
        if w is not None:
            v = w[:wv * body].view(vecs, wv, 4)
            for i in range(wv):
                assert torch.equal(v[:, i, 0], lane) and (v[:, i, 1] == groups - 1).all()
                assert not v[:, i, 2:].any()
