"""GPU parity of the downstream measurement of a decode step: the vocabulary
projection (bit-exact against the oracle, same pinned order), the fp32
log-softmax (bit-exact: the same fp32 steps with correctly rounded exp and log
on both sides; also within the bound of its fixed chunked sums) and k3 (fp64),
plus their batch invariance on the decode configuration."""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special as sps
import torch

from helpers import DEV, bits, gpu, layer, log
from oracle import oracle as O
from serve_router_gemm_amd import inputs as I
from serve_router_gemm_amd import moe as M

pytestmark = gpu
U = 2.0 ** -24
V_DEC = 65536

_proj = {}


def proj(H, V=V_DEC):
    """The downstream projection [V, H] bf16 from its own seed (CPU generator,
    so its bytes do not depend on the device)."""
    if (H, V) not in _proj:
        g = torch.Generator().manual_seed(I.PROJ_SEED)
        _proj[(H, V)] = torch.randn((V, H), generator=g).to(torch.bfloat16).to(DEV)
    return _proj[(H, V)]


def _ls_bound(z, logp, chunk=256):
    V = z.shape[-1]
    nch = (V + chunk - 1) // chunk
    m = z.max(axis=-1, keepdims=True).astype(np.float64)
    lnS = sps.logsumexp(z.astype(np.float64) - m, axis=-1, keepdims=True)
    rel = (min(chunk, V) - 1 + nch + 2) * U
    return rel + U * (np.abs(lnS) + np.abs(m + lnS) + np.abs(logp.astype(np.float64))) + 1e-12


@pytest.mark.parametrize("T,H,V", [(5, 512, 3001), (1, 64, 1), (9, 256, 257)])
def test_lm_head_logits_bit_exact_small(T, H, V):
    g = torch.Generator().manual_seed(T * 1000 + V)
    h = torch.randn((T, H), generator=g).to(torch.bfloat16)
    p = (torch.randn((V, H), generator=g) * 0.05).to(torch.bfloat16)
    z = M.lm_head_logits(h.to(DEV), p.to(DEV)).cpu().numpy()
    ref = O.lm_head_logits(bits(h), bits(p))
    assert np.array_equal(z.view(np.uint32), ref.view(np.uint32))


def _dec_outputs(n):
    """Layer outputs of n probe tokens of the decode configuration, each alone."""
    cfg = I.CONFIGS["dec"]
    L = layer(cfg)
    pr = I.probes(cfg.H, n, DEV)
    outs = [M.forward(pr[i:i + 1].contiguous(), L["w_router"], L["w_gate"], L["w_up"],
                      L["w_down"], cfg.k, cfg.score, cfg.renorm, bias=L["bias"])
            for i in range(n)]
    return cfg, L, torch.cat(outs, 0)


def test_decode_projection_logsoftmax_k3_parity():
    """Decode shapes (H = 6144, V = 65536): z and logp bit-exact, k3 within
    fp64 rounding of the oracle on the same inputs."""
    cfg, L, h = _dec_outputs(3)
    P = proj(cfg.H)
    z = M.lm_head_logits(h, P)
    logp = M.log_softmax(z)
    zc = z.cpu().numpy()
    log(f"[decode-measure] projecting {h.shape[0]} outputs onto {V_DEC} rows on the CPU")
    zr = O.lm_head_logits(bits(h), bits(P))
    assert np.array_equal(zc.view(np.uint32), zr.view(np.uint32))
    lg = logp.cpu().numpy()
    lr = O.log_softmax(zc)
    err = np.abs(lg.astype(np.float64) - lr.astype(np.float64))
    same = float(np.mean(lg.view(np.uint32) == lr.view(np.uint32)))
    log(f"[decode-measure] logp max |gpu - oracle| {err.max():.3e}, bit-identical {same:.6f}")
    # both sides take the same fp32 steps with correctly rounded exp and log
    assert np.array_equal(lg.view(np.uint32), lr.view(np.uint32)), \
        f"{int((lg.view(np.uint32) != lr.view(np.uint32)).sum())} logp differ"
    # k3 between two different tokens' distributions (a large KL), same inputs
    ref_rows, test_rows = logp[[0, 1]].contiguous(), logp[[1, 2]].contiguous()
    mean, gk3, g = M.k3(ref_rows, test_rows)
    om, ogk3, og = O.k3(ref_rows.cpu().numpy(), test_rows.cpu().numpy())
    assert np.array_equal(g.cpu().numpy(), og)
    assert np.allclose(mean.cpu().numpy(), om, rtol=1e-9, atol=1e-15)
    assert np.allclose(gk3.cpu().numpy(), ogk3, rtol=1e-9, atol=1e-15)
    # and against the library's generalized KL divergence
    pr = np.exp(ref_rows.cpu().numpy().astype(np.float64))
    pt = np.exp(test_rows.cpu().numpy().astype(np.float64))
    assert np.allclose(mean.cpu().numpy(), sps.kl_div(pt, pr).sum(-1), rtol=1e-9)


def test_k3_random_rows_and_edge_cases():
    rng = np.random.default_rng(4)
    for V in (1, 2, 255, 257, 4096):
        a = O.log_softmax((rng.standard_normal((3, V)) * 2).astype(np.float32))
        b = O.log_softmax((rng.standard_normal((3, V)) * 2).astype(np.float32))
        mean, gk3, g = M.k3(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
        om, ogk3, og = O.k3(a, b)
        assert np.array_equal(g.cpu().numpy(), og), V
        assert np.allclose(mean.cpu().numpy(), om, rtol=1e-9, atol=1e-15), V
        assert np.allclose(gk3.cpu().numpy(), ogk3, rtol=1e-9, atol=1e-15), V
        z0, _, _ = M.k3(torch.from_numpy(a).to(DEV), torch.from_numpy(a).to(DEV))
        assert np.all(z0.cpu().numpy() == 0.0)
    # greedy: ties take the lowest index; a NaN at 0 gives 0; other NaNs skipped
    t = np.log(np.array([[0.1, 0.4, 0.1, 0.4], [0.2, 0.2, 0.3, 0.3]], dtype=np.float32))
    t[1, 2] = np.nan
    r = np.log(np.full((2, 4), 0.25, dtype=np.float32))
    _, _, g = M.k3(torch.from_numpy(r).to(DEV), torch.from_numpy(t).to(DEV))
    _, _, og = O.k3(r, t)
    assert g.cpu().tolist() == [1, 3] and og.tolist() == [1, 3]
    t[0, 0] = np.nan
    _, _, g = M.k3(torch.from_numpy(r).to(DEV), torch.from_numpy(t).to(DEV))
    _, _, og = O.k3(r, t)
    assert g.cpu().tolist()[0] == 0 and og.tolist()[0] == 0
    # ties far apart (other waves of the block) and in one thread's elements
    V = 70000
    t = O.log_softmax((rng.standard_normal((3, V))).astype(np.float32))
    r = O.log_softmax((rng.standard_normal((3, V))).astype(np.float32))
    t[0, [61000, 3000, 45000]] = 0.0           # across waves: 3000 wins
    t[1, [2048, 1024, 3072]] = 0.0             # one thread's elements: 1024 wins
    t[2, [7, 69999]] = 0.0
    t[2, 5] = -0.0                              # -0 == +0: 5 wins
    _, _, g = M.k3(torch.from_numpy(r).to(DEV), torch.from_numpy(t).to(DEV))
    _, _, og = O.k3(r, t)
    assert g.cpu().tolist() == [3000, 1024, 5] and og.tolist() == [3000, 1024, 5]


def test_log_softmax_in_place_and_edge_rows():
    rng = np.random.default_rng(8)
    for V in (1, 3, 256, 1000, 65537):
        z = (rng.standard_normal((2, V)) * 5).astype(np.float32)
        z[1] = 0.0
        zt = torch.from_numpy(z).to(DEV)
        out = M.log_softmax(zt)
        M.log_softmax(zt, out=zt)            # in place
        assert torch.equal(out, zt)
        lr = O.log_softmax(z)
        lg = out.cpu().numpy()
        err = np.abs(lg.astype(np.float64) - lr.astype(np.float64))
        assert np.all(err <= 2 * _ls_bound(z, lr)), V
        assert np.array_equal(lg.view(np.uint32), lr.view(np.uint32)), V
        assert np.all(lg[1] == lg[1, 0])     # constant row: one value


def test_decode_logprobs_batch_invariant():
    """The probe's log-probabilities are bit-identical at T in {1, 4, 16, 64}
    (fresh co-tokens each step, the probe in the middle), so k3 is exactly 0."""
    cfg = I.CONFIGS["dec"]
    L = layer(cfg)
    P = proj(cfg.H)
    probe = I.probes(cfg.H, 1, DEV)
    o1 = M.forward(probe, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score,
                   cfg.renorm, bias=L["bias"])
    ref = M.log_softmax(M.lm_head_logits(o1, P))
    for T in I.DEC_SWEEP_T:
        x = I.make_tokens(T, cfg.H, I.COTOKEN_SEED_BASE + 29 * T, "cpu").to(DEV)
        x[T // 2] = probe[0]
        o = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score,
                      cfg.renorm, bias=L["bias"])
        lp = M.log_softmax(M.lm_head_logits(o, P))
        assert torch.equal(lp[T // 2:T // 2 + 1].view(torch.int32), ref.view(torch.int32)), T
        mean, gk3, _ = M.k3(ref, lp[T // 2:T // 2 + 1].contiguous())
        assert mean.item() == 0.0 and gk3.item() == 0.0
    log("[decode-measure] probe log-probs bit-identical at T = 1, 4, 16, 64; k3 = 0")
