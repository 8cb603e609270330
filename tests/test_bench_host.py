"""Host logic of bench.py, on the CPU: the algorithmic byte count the
headline divides by, the kernel-source hash that decides whether the
committed counter traffic still applies, the traffic it reads, and the
one-GPU guard."""
import importlib.util
import json
import pathlib
import re
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_match_the_per_element_count(bench):
    # every rank buffer read once and written once, w read once and written once
    assert bench.alg_bytes(10, 300_000_000, 4, True) == 26_400_000_000
    assert bench.alg_bytes(40, 100_000_000, 2, True) == 16_800_000_000
    assert bench.alg_bytes(4, 1_000_003, 4, False) == 2 * 4 * 1_000_003 * 4
    assert bench.alg_bytes(1, 0, 4, True) == 0


def test_kernel_hash_ignores_comments_and_whitespace_only(bench, tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) { return x + 1; }  // one\n/* two */\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", src)
    h0 = bench.kernel_sha()
    src.write_text("// a new comment\nint f(int x)\n{\n    return x + 1;  /* spread out */\n}\n")
    assert bench.kernel_sha() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_sha() != h0


@pytest.mark.parametrize("workload,dtype,alg", [("n10_p300m_f32_sgd", "f32", 26_400_000_000),
                                                ("n40_p100m_bf16_sgd", "bf16", 16_800_000_000)])
def test_committed_traffic_is_read_only_for_the_current_kernel(bench, monkeypatch, workload, dtype, alg):
    f = ROOT / "profiles" / f"fused_{dtype}_sgd_{workload}_pmc.md"
    d = json.loads(re.search(r"```json\s*(\{.*?\})\s*```", f.read_text(), re.S).group(1))
    traffic = bench.committed_traffic(workload, dtype)
    if d["kernel_src_sha256_16"] == bench.kernel_sha():
        # the summary was taken on the current kernel code: its bytes, close to the algorithm's
        assert traffic == d["hbm_bytes_per_launch"]
        assert abs(traffic / alg - 1) < 0.01
    else:
        assert traffic is None
    monkeypatch.setattr(bench, "kernel_sha", lambda: "0" * 16)
    assert bench.committed_traffic(workload, dtype) is None
    assert bench.committed_traffic("no_such_workload", dtype) is None


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in (r.stdout + r.stderr)
