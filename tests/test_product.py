"""Host-side properties of the product path (CPU): it never reaches the
oracle, it fails loudly without its HIP library, and the benchmark refuses
more than one GPU before touching any."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_top_decode_query_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            yield node.module


def test_package_never_imports_the_oracle():
    for name in os.listdir(PKG):
        if name.endswith(".py"):
            mods = list(_imports(os.path.join(PKG, name)))
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), name


def test_missing_library_raises():
    from sparse_top_decode_query_amd import lib
    saved = lib._lib
    lib._lib = None
    try:
        with pytest.raises(lib.SDQError):
            lib.load(os.path.join(ROOT, "no_such_dir", "libsdq.so"))
    finally:
        lib._lib = saved


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
