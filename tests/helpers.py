"""Shared helpers of the GPU tests: cached layers, host copies for the oracle,
and the comparison rules.

Comparison rules (the layer's contract):
  * integers (expert ids, counts, offsets, perm, inv_perm): bit-exact, except
    tokens whose k-th/(k+1)-th key gap (from the oracle, in fp64) is below
    1e-6: those are counted and reported, and excluded from value checks;
  * out (bf16): |gpu - ref| <= 2e-2 + 1e-2*|ref| per element;
  * stages fed the GPU's own inputs: combine bit-exact; down projection within
    the fp32 summation bound gamma_F * sum|act*w|; gate/up act within the
    derived bound of the fp32 sums plus one bf16 ulp.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

DEV = "cuda"
GAP_EXEMPT = 1e-6
ATOL, RTOL = 2e-2, 1e-2
U32 = 2.0 ** -24

gpu = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return I.bf16_bits(t)


def f32(b: np.ndarray) -> np.ndarray:
    return O.bf16_to_f32(b)


_layers: dict = {}
_host: dict = {}


def layer(cfg: I.LayerConfig) -> dict:
    """Layer weights on the GPU, cached per layer shape and seed."""
    key = (cfg.H, cfg.E, cfg.F, cfg.score, cfg.w_std, cfg.seed, cfg.zipf_s, cfg.kappa)
    if key not in _layers:
        log(f"[layer] generating {I.describe(cfg)} on {DEV}")
        _layers[key] = I.make_layer(cfg, DEV)
        torch.cuda.synchronize()
    return _layers[key]


def host(cfg: I.LayerConfig) -> dict:
    """uint16 / fp32 host copies of layer(cfg), for the oracle."""
    key = (cfg.H, cfg.E, cfg.F, cfg.score, cfg.w_std, cfg.seed, cfg.zipf_s, cfg.kappa)
    if key not in _host:
        L = layer(cfg)
        _host[key] = {n: (bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy())
                      for n, t in L.items() if t is not None}
        _host[key]["bias"] = L["bias"].cpu().numpy() if L["bias"] is not None else None
    return _host[key]


def routing_compare(ids_gpu, ids_ref, gap_ref, exempt_ok=True, strict_rows=None):
    """Bit-exact ids except rows with gap < 1e-6.  Returns (n_exempt, n_mismatch_exempt)."""
    ids_gpu = np.asarray(ids_gpu)
    ids_ref = np.asarray(ids_ref)
    diff = np.any(ids_gpu != ids_ref, axis=1)
    exempt = gap_ref < GAP_EXEMPT
    if strict_rows is not None:
        exempt = exempt & ~strict_rows
    bad = diff & ~exempt
    assert not bad.any(), (f"{int(bad.sum())} non-exempt routing mismatches, first rows "
                           f"{np.nonzero(bad)[0][:8].tolist()}")
    return int(exempt.sum()), int((diff & exempt).sum())


def assert_out_close(gpu_bits, ref_bits, what="out", rows=None):
    g = f32(np.asarray(gpu_bits)).astype(np.float64)
    r = f32(np.asarray(ref_bits)).astype(np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    err = np.abs(g - r)
    lim = ATOL + RTOL * np.abs(r)
    ok = err <= lim
    same = float(np.mean(np.asarray(gpu_bits)[rows] == np.asarray(ref_bits)[rows])
                 if rows is not None else np.mean(np.asarray(gpu_bits) == np.asarray(ref_bits)))
    stats = dict(max_abs=float(err.max()) if err.size else 0.0,
                 max_rel=float((err / np.maximum(np.abs(r), 1e-30)).max()) if err.size else 0.0,
                 bit_identical=same, n=int(err.size))
    assert ok.all(), f"{what}: {int((~ok).sum())} elements out of tolerance; {stats}"
    return stats


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (for normal numbers)."""
    a = np.abs(v).astype(np.float32)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def weights_close(w_gpu, w_ref, rel=1e-5):
    w_gpu = np.asarray(w_gpu, np.float64)
    w_ref = np.asarray(w_ref, np.float64)
    assert np.all(np.abs(w_gpu - w_ref) <= rel * np.abs(w_ref) + 1e-9), \
        f"weights differ: max {np.max(np.abs(w_gpu - w_ref))}"
