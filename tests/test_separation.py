"""The product path and the oracle stay apart, and the product has no
fallback: both checked without a GPU."""
import pathlib
import re
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]
PKG = ROOT / "ring_all_reduce_amd"


def test_binding_raises_when_the_library_is_missing():
    code = (
        "import pathlib, ring_all_reduce_amd._lib as L\n"
        "L.LIB_PATH = pathlib.Path('/nonexistent/librar.so')\n"
        "from ring_all_reduce_amd import api\n"
        "try:\n"
        "    api.rar_version()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    raise SystemExit('no error without the library')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised:" in r.stdout and "no fallback" in r.stdout


def test_product_sources_do_not_touch_the_oracle():
    bad = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b|.*ring_oracle|.*libring_oracle)", re.M)
    for f in list(PKG.rglob("*.py")) + list(PKG.rglob("*.hip")) + list(PKG.rglob("*.cpp")) + list(PKG.rglob("*.h")):
        assert not bad.search(f.read_text()), f"{f} refers to the oracle"


def test_oracle_does_not_use_the_product():
    for f in (ROOT / "oracle").rglob("*"):
        if f.suffix not in (".py", ".c", ".h"):
            continue
        text = f.read_text()
        assert not re.search(r"^\s*(import|from)\s+ring_all_reduce_amd", text, re.M), f"{f} imports the product"
        assert not re.search(r'#include\s+[<"](rar|rar_internal)\.h[>"]', text), f"{f} includes a library header"
        assert not re.search(r"librar\.so", text), f"{f} loads the library"
