"""The product path's separation from the oracle, and its refusals (CPU only).

The package and the input generators never import the oracle; bench.py
imports it only inside its CPU-baseline functions; the package raises when
the HIP library is missing; bench.py refuses more than one GPU.
"""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(tree):
    """(module name, enclosing function name or None) for every import."""
    out = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import):
                out.extend((a.name, fn) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append(((child.module or "") if child.level == 0 else "." + (child.module or ""), fn))
            visit(child, f)

    visit(tree, None)
    return out


def _py_files(*dirs):
    for d in dirs:
        for dp, _, fs in os.walk(os.path.join(ROOT, d)):
            for f in fs:
                if f.endswith(".py"):
                    yield os.path.join(dp, f)


def test_package_and_generators_never_import_the_oracle():
    files = list(_py_files("lm_head_cross_amd", "workloads"))
    assert files
    for path in files:
        with open(path) as fh:
            src = fh.read()
        for mod, _ in _imports(ast.parse(src)):
            assert mod.split(".")[0] != "oracle", f"{path} imports {mod}"
        assert "importlib" not in src and "__import__" not in src, f"{path} imports dynamically"


def test_bench_imports_the_oracle_only_in_its_cpu_baseline_legs():
    with open(os.path.join(ROOT, "bench.py")) as fh:
        tree = ast.parse(fh.read())
    legs = [fn for mod, fn in _imports(tree) if mod.split(".")[0] == "oracle"]
    assert legs, "the CPU baseline legs import the oracle"
    assert all(fn is not None and "cpu_baseline" in fn for fn in legs), legs


def test_hip_sources_do_not_include_oracle_code():
    csrc = os.path.join(ROOT, "lm_head_cross_amd", "csrc")
    for f in os.listdir(csrc):
        with open(os.path.join(csrc, f)) as fh:
            src = fh.read()
        for line in src.splitlines():
            if line.lstrip().startswith("#include"):
                assert "oracle" not in line, f"{f}: {line}"


def test_missing_library_raises(monkeypatch, tmp_path):
    from lm_head_cross_amd import _lib

    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libflce.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""
