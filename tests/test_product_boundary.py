"""Host-side checks of the product boundary (no GPU needed).

The benchmark refuses more than one GPU; the HIP package never reaches the
CPU oracle (only tests, the smoke check and the benchmark's CPU baseline
may); and the binding fails loudly when the HIP library is missing instead of
computing anything elsewhere.
"""
from __future__ import annotations

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "serve_router_gemm_amd")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def _imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if name.endswith(".py"):
            mods = list(_imported_modules(os.path.join(PKG, name)))
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_binding_fails_loudly_without_the_library():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from serve_router_gemm_amd import moe as M\n"
        "M.LIB_PATH = '/nonexistent/libmoe.so'\n"
        "M._lib = None\n"
        "try:\n"
        "    M.lib()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('no error')\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "missing" in r.stdout
