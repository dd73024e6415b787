"""Properties of the compiled gfx950 code that the batch-invariance argument
and the performance design rely on (no GPU needed: hipcc cross-compiles)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from serve_router_gemm_amd import build as B

HIPCC = B.HIPCC
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def _device_compile(src: str, extra=()):
    cmd = [HIPCC, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(B.ROOT, "include"), "--cuda-device-only", *extra, src]
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _resources():
    out = {}
    for src in B.sources():
        r = _device_compile(src, ["-c", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"])
        assert r.returncode == 0, r.stdout[-2000:]
        name = None
        for line in r.stdout.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                out[name] = {}
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
            if m and name:
                out[name][m.group(1).strip()] = int(m.group(2))
    return out


def test_no_scratch_and_expert_gemm_occupancy():
    res = _resources()
    assert res, "no kernels found"
    for name, r in res.items():
        assert r.get("ScratchSize", 0) == 0, (name, r)
        if "expert_gemm" in name:
            assert r["VGPRs"] + r.get("AGPRs", 0) <= 256, (name, r)
            assert r["Occupancy"] >= 2, (name, r)


def test_expert_gemm_uses_one_mfma_instruction(tmp_path):
    """Every MFMA the expert GEMMs can execute is v_mfma_f32_16x16x32_bf16:
    no remainder path with another instruction exists."""
    src = os.path.join(B.PKG, "csrc", "moe_gemm.hip")
    asm = tmp_path / "gemm.s"
    r = _device_compile(src, ["-S", "-o", str(asm)])
    assert r.returncode == 0, r.stdout[-2000:]
    text = asm.read_text()
    ops = set(re.findall(r"\b(v_mfma_\w+)", text))
    assert ops == {"v_mfma_f32_16x16x32_bf16"}, ops
