"""Host-side checks of the product boundary (no GPU): the package never reaches the oracle, the
binding fails loudly without its library, and the benchmark's command line keeps its contract."""

import ast
import os
import subprocess
import sys

import pytest

import sparse_long_context_lightning_amd as dsa
from sparse_long_context_lightning_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_long_context_lightning_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    names = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names += [a.name for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            names.append(node.module or "")
    return names


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith(".py"):
                mods = _imports(os.path.join(dirpath, f))
                assert not any(m.split(".")[0] in ("oracle", "dsa_oracle", "dsa_testlib") for m in mods), f


def test_benchmark_imports_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for fn in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        mods = [m for node in ast.walk(fn) if isinstance(node, (ast.Import, ast.ImportFrom))
                for m in ([a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""])]
        if any(m.split(".")[0] in ("oracle", "dsa_testlib") for m in mods):
            assert fn.name == "cpu_baseline", fn.name
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    for node in top:
        mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
        assert not any(m.split(".")[0] in ("oracle", "dsa_testlib") for m in mods)


def test_binding_raises_without_its_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(PKG, "no_such_libdsa.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.load()


def test_library_is_the_in_tree_build():
    assert os.path.dirname(os.path.abspath(dsa.LIB_PATH)) == PKG


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_bench_defaults_finish_in_minutes():
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.gpus == 1 and args.steps == 5 and args.warmup == 1
