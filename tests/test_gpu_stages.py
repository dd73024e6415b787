"""Per-stage parity of the HIP path against the CPU oracle (GPU required).

Each stage is fed its inputs from the previous GPU stage, so a failure names
one kernel: route (ids bit-exact, weights to a few ulp), permute (bit-exact),
gate/up (act codes within the bound the fp32 sums allow), down (within the fp32 summation
bound), combine (bit-exact).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import (DEV, GAP_EXEMPT, U32, bf16_ulp, bits, f32, gpu, host, layer, log,
                     routing_compare, weights_close)
from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

pytestmark = gpu

if torch.cuda.is_available():
    from serve_router_gemm_amd import moe as M


def _cfg(name, **kw):
    return I.scaled(I.CONFIGS[name], **kw)


# (config, T, rows compared with the oracle (None = all))
ROUTE_CASES = [
    ("tiny", _cfg("tiny"), None),
    ("mid_T7", _cfg("mid", T=7), None),
    ("mid_T1024", _cfg("mid", T=1024), 256),
    ("mid_T4096", _cfg("mid", T=4096), 256),
    ("large_T16384", _cfg("large"), 512),
    ("dec_T1", _cfg("dec", T=1), None),
    # up to 8 tokens: one wave per (256-wide chunk, 64 experts), 1/2/4/8 token
    # chains per thread
    ("mid_T2_few", _cfg("mid", T=2), None),
    ("dec_T3_few", _cfg("dec", T=3), None),
    ("dec_T8_few", _cfg("dec", T=8), None),
    ("dec_T64", _cfg("dec", T=64), None),
    ("E512_k16_H320", _cfg("mid", T=300, E=512, k=16, H=320, F=128), None),
    ("kE_E8", _cfg("tiny", T=50, k=8), None),
    ("E1_k1", _cfg("tiny", T=33, E=1, k=1), None),
    ("sigmoid_norenorm", _cfg("large", T=200, H=512, E=64, renorm=False), None),
    # the matrix-core logits kernel, one block per chunk: a ragged token block
    # (600 = 4 x 128 + 88) and a last chunk 64 wide (H = 52 x 256 + 64)
    ("mfma_split_ragged", _cfg("mid", T=600, H=13376, F=128), 256),
    # the matrix-core kernel folding every chunk: ragged token and expert
    # blocks (16400 = 256 x 64 + 16 tokens, 200 = 128 + 72 experts)
    ("mfma_fold_ragged", _cfg("large", T=16400, H=256, E=200, F=128), 512),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: c[0])
def test_route_parity(case):
    name, cfg, nsample = case
    log(f"[route] {name}: {I.describe(cfg)}")
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    ids, w = M.route(x, L["w_router"], cfg.k, cfg.score, cfg.renorm, bias=L["bias"])
    torch.cuda.synchronize()
    rows = np.arange(cfg.T)
    if nsample is not None and nsample < cfg.T:
        rows = np.sort(np.random.default_rng(1).choice(cfg.T, nsample, replace=False))
    hb = host(cfg)
    xr = bits(x)[rows]
    ids_r, w_r, gap = O.route(xr, hb["w_router"], cfg.k, cfg.score, cfg.renorm, bias=hb["bias"])
    ids_g = ids.cpu().numpy()[rows]
    w_g = w.cpu().numpy()[rows]
    n_ex, n_ex_mis = routing_compare(ids_g, ids_r, gap)
    ok = np.all(ids_g == ids_r, axis=1)
    weights_close(w_g[ok], w_r[ok])
    log(f"[route] {name}: rows={len(rows)} exempt={n_ex} exempt_mismatch={n_ex_mis}")
    if cfg.score == I.SCORE_SOFTMAX:
        # softmax keys are the logits, taken in the same fixed fp32 order on
        # both sides: even near-ties must agree
        assert n_ex_mis == 0


def test_route_tie_stress_full():
    """Constructed exact ties and 1-ulp gaps: every stress token bit-exact, no exemption."""
    cfg = I.CONFIGS["tie"]
    d = I.make_tie_inputs(cfg)
    wr = d["w_router"].to(DEV)
    x = d["x"].to(DEV)
    ids, w = M.route(x, wr, cfg.k, cfg.score, cfg.renorm)
    torch.cuda.synchronize()
    ids_r, w_r, gap = O.route(bits(d["x"]), bits(d["w_router"]), cfg.k, cfg.score, cfg.renorm)
    stress = d["kind"] >= 2
    n_ex, n_mis = routing_compare(ids.cpu().numpy(), ids_r, gap, strict_rows=stress)
    assert np.array_equal(ids.cpu().numpy()[stress], ids_r[stress])
    weights_close(w.cpu().numpy(), w_r)
    log(f"[route] tie: T={cfg.T} stress={int(stress.sum())} exempt(random rows)={n_ex} "
        f"mismatch={n_mis}")


def test_route_nan_and_inf_rows():
    """NaN / inf hidden states: ids follow the NaN-last rule and match the oracle."""
    cfg = _cfg("tiny", T=16)
    L = layer(cfg)
    x = I.make_x(cfg, "cpu")
    x[3, 5] = float("nan")       # every logit NaN -> ids 0..k-1
    x[4, :] = float("inf")       # +-inf / NaN mixture
    x[5, 7] = float("-inf")
    xd = x.to(DEV)
    ids, w = M.route(xd, L["w_router"], cfg.k, cfg.score, cfg.renorm)
    ids_r, w_r, gap = O.route(bits(x), host(cfg)["w_router"], cfg.k, cfg.score, cfg.renorm)
    assert np.array_equal(ids.cpu().numpy(), ids_r)
    assert ids.cpu().numpy()[3].tolist() == list(range(cfg.k))


# ---------------------------------------------------------------------------
# permute
# ---------------------------------------------------------------------------

def _ids_cases():
    rng = np.random.default_rng(4)
    yield "tiny_random", rng.integers(0, 8, size=(64, 2)), 8
    yield "T1", np.array([[5, 1, 7]]), 8
    yield "all_one_expert", np.zeros((3000, 1), dtype=np.int64), 16
    yield "skewed_E512", (rng.zipf(1.3, size=(5000, 4)) - 1) % 512, 512
    yield "ragged_A", rng.integers(0, 64, size=(1237, 8)), 64
    yield "large_A", rng.integers(0, 256, size=(16384, 8)), 256
    yield "multi_chunk_2M", rng.integers(0, 128, size=(262144, 8)), 128


@pytest.mark.parametrize("case", list(_ids_cases()), ids=lambda c: c[0])
def test_permute_parity(case):
    name, ids_np, E = case
    ids_np = np.ascontiguousarray(ids_np, dtype=np.int32)
    log(f"[permute] {name}: T={ids_np.shape[0]} k={ids_np.shape[1]} E={E}")
    ids = torch.from_numpy(ids_np).to(DEV)
    counts, offsets, perm, inv = M.permute(ids, E)
    torch.cuda.synchronize()
    c_r, o_r, p_r, i_r = O.permute(ids_np, E)
    assert np.array_equal(counts.cpu().numpy(), c_r)
    assert np.array_equal(offsets.cpu().numpy(), o_r)
    assert np.array_equal(perm.cpu().numpy(), p_r)
    assert np.array_equal(inv.cpu().numpy(), i_r)


def test_permute_skips_invalid_ids():
    rng = np.random.default_rng(6)
    ids_np = rng.integers(0, 16, size=(500, 4)).astype(np.int32)
    bad = rng.random(ids_np.shape) < 0.1
    ids_np[bad] = rng.choice([-1, 16, 1000], size=int(bad.sum()))
    ids = torch.from_numpy(ids_np).to(DEV)
    counts, offsets, perm, inv = M.permute(ids, 16)
    flat = ids_np.reshape(-1)
    valid = (flat >= 0) & (flat < 16)
    c_r, o_r, p_r, _ = O.permute(np.where(valid, flat, 0)[valid], 16)
    A_valid = int(valid.sum())
    assert np.array_equal(counts.cpu().numpy(), c_r)
    assert offsets.cpu().numpy()[-1] == A_valid
    # valid assignments in stable order by expert
    idx_valid = np.nonzero(valid)[0]
    assert np.array_equal(perm.cpu().numpy()[:A_valid], idx_valid[p_r])
    inv_g = inv.cpu().numpy()
    assert np.all(inv_g[~valid] == -1)
    assert np.array_equal(perm.cpu().numpy()[inv_g[valid]], idx_valid)


# ---------------------------------------------------------------------------
# expert GEMMs
# ---------------------------------------------------------------------------

GEMM_CASES = [
    ("tiny", _cfg("tiny")),
    ("mid_T300", _cfg("mid", T=300)),
    ("mid_T7", _cfg("mid", T=7)),
    ("Fedge_Hedge", _cfg("mid", T=257, H=320, F=192, E=16, k=4)),
    # every expert far below 64 tokens: the gate/up launch keeps two steps of
    # loads in flight, here over 5 K steps (not a multiple of its 3 stages)
    ("Hedge_streaming", _cfg("mid", T=40, H=320, F=192, E=16, k=4)),
    ("E1_k1", _cfg("tiny", T=300, E=1, k=1)),
    # batches of at most 32 tokens run the weight-streaming kernel: 16-row and
    # 32-row token chunks, rings of 8, 4 (F = 1408) and 2 (H = 320, F = 192)
    # K steps, one expert holding every token
    ("mid_T20_stream", _cfg("mid", T=20)),
    ("Hedge_stream_ring2", _cfg("mid", T=24, H=320, F=192, E=16, k=4)),
    ("dec_T5_stream", _cfg("dec", T=5)),
    ("E1_k1_T3_stream", _cfg("tiny", T=3, E=1, k=1)),
]


def _routed(cfg, x, L):
    ids, w = M.route(x, L["w_router"], cfg.k, cfg.score, cfg.renorm, bias=L["bias"])
    counts, offsets, perm, inv = M.permute(ids, cfg.E)
    return ids, w, counts, offsets, perm


def act_bound(cfg, hb, xb, tok, exp_):
    """Largest |act_gpu - act_exact| the arithmetic allows before bf16 rounding.

    g and u are fp32 sums of H exact products in some order: |dg| <= gamma_H *
    sum|x*w_gate| (any summation order), the same for u.  silu' is at most
    1.1 in magnitude, and the fp32 evaluation of silu(g)*u adds at most 8
    roundings relative to the result.
    """
    H = cfg.H
    gamma = H * U32 / (1 - H * U32)
    xd = f32(xb).astype(np.float64)
    out = np.empty((tok.size, cfg.F), dtype=np.float64)
    for e in np.unique(exp_):
        rows = exp_ == e
        xe = xd[tok[rows]]
        wg = f32(hb["w_gate"][e]).astype(np.float64)
        wu = f32(hb["w_up"][e]).astype(np.float64)
        g, u = xe @ wg.T, xe @ wu.T
        dg, du = gamma * (np.abs(xe) @ np.abs(wg).T), gamma * (np.abs(xe) @ np.abs(wu).T)
        sg = g / (1.0 + np.exp(-g))
        out[rows] = 1.1 * dg * (np.abs(u) + du) + np.abs(sg) * du + 8 * U32 * np.abs(sg * u)
    return out


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: c[0])
def test_gate_up_and_down_parity(case):
    name, cfg = case
    log(f"[gemm] {name}: {I.describe(cfg)}")
    L = layer(cfg)
    hb = host(cfg)
    x = I.make_x(cfg, DEV)
    ids, w, counts, offsets, perm = _routed(cfg, x, L)
    h_act = M.expert_gate_up(x, perm, offsets, L["w_gate"], L["w_up"], cfg.k)
    y = M.expert_down(h_act, perm, offsets, L["w_down"], cfg.k)
    torch.cuda.synchronize()
    perm_np = perm.cpu().numpy()
    offs = offsets.cpu().numpy()
    A = cfg.T * cfg.k
    exp_of_p = np.searchsorted(offs, np.arange(A), side="right") - 1
    tok_of_p = perm_np // cfg.k

    # gate/up: act codes vs the oracle's, same (token, expert) pairs
    y_ref_full, act_ref = O.expert_ffn(tok_of_p, exp_of_p, bits(x), hb["w_gate"], hb["w_up"],
                                       hb["w_down"], want_act=True)
    act_g = bits(h_act)
    a_g = f32(act_g).astype(np.float64)
    a_r = f32(act_ref).astype(np.float64)
    diff = np.abs(a_g - a_r)
    lim = act_bound(cfg, hb, bits(x), tok_of_p, exp_of_p) + bf16_ulp(np.maximum(np.abs(a_g),
                                                                           np.abs(a_r)))
    assert np.all(diff <= lim), f"act: max diff {diff.max()}, worst ratio {np.max(diff / lim)}"
    frac_same = float(np.mean(act_g == act_ref))
    assert frac_same > 0.95, frac_same

    # down on the GPU's own act codes: fp32 summation bound gamma_F * sum|a*w|
    y_ref = O.expert_down(exp_of_p, act_g, hb["w_down"])
    y_g = y.cpu().numpy()[perm_np]         # y is in assignment order; bring to perm order
    wd = hb["w_down"]
    absum = np.empty_like(y_ref, dtype=np.float64)
    for e in np.unique(exp_of_p):
        rows = exp_of_p == e
        absum[rows] = np.abs(a_g[rows]) @ np.abs(f32(wd[e]).astype(np.float64)).T
    gamma = cfg.F * U32 / (1 - cfg.F * U32)
    err = np.abs(y_g.astype(np.float64) - y_ref)
    assert np.all(err <= gamma * absum + np.abs(y_ref) * U32), f"down: max err {err.max()}"
    log(f"[gemm] {name}: act same={frac_same:.5f} max|dy|={err.max():.3e} "
        f"(bound ratio {np.max(err / np.maximum(gamma * absum, 1e-30)):.3f})")


def test_down_splitk_variant_close_but_not_invariant_path():
    """The split-K variant still computes the down projection (within the bound)."""
    cfg = _cfg("mid", T=64)
    L = layer(cfg)
    hb = host(cfg)
    x = I.make_x(cfg, DEV)
    ids, w, counts, offsets, perm = _routed(cfg, x, L)
    h_act = M.expert_gate_up(x, perm, offsets, L["w_gate"], L["w_up"], cfg.k)
    y_inv = M.expert_down(h_act, perm, offsets, L["w_down"], cfg.k, variant=M.INVARIANT)
    y_var = M.expert_down(h_act, perm, offsets, L["w_down"], cfg.k, variant=M.SPLITK_VARIANT)
    torch.cuda.synchronize()
    a, b = y_inv.cpu().numpy(), y_var.cpu().numpy()
    scale = np.abs(a).max()
    assert np.max(np.abs(a - b)) <= 1e-5 * scale
    log(f"[gemm] split-K variant: {np.mean(a != b):.3f} of y elements differ in bits")


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

def test_combine_bit_exact_random():
    rng = np.random.default_rng(8)
    for T, H, k in [(1, 64, 1), (37, 320, 8), (513, 2048, 8), (64, 256, 16)]:
        y = rng.standard_normal((T * k, H)).astype(np.float32) * 3
        w = rng.random((T, k)).astype(np.float32)
        y[0, :5] = [np.inf, -np.inf, np.nan, 3e38, -0.0]
        out = M.combine(torch.from_numpy(y).to(DEV), torch.from_numpy(w).to(DEV))
        ref = O.combine(y, w, T, H, k)
        g = bits(out)
        nan = np.isnan(f32(ref))
        assert np.array_equal(np.isnan(f32(g)), nan)
        assert np.array_equal(g[~nan], ref[~nan]), (T, H, k)


def test_combine_bit_exact_on_pipeline():
    cfg = _cfg("mid", T=129)
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    ids, w, counts, offsets, perm = _routed(cfg, x, L)
    y = M.grouped_swiglu(x, perm, offsets, L["w_gate"], L["w_up"], L["w_down"], cfg.k)
    out = M.combine(y, w)
    ref = O.combine(y.cpu().numpy(), w.cpu().numpy(), cfg.T, cfg.H, cfg.k)
    assert np.array_equal(bits(out), ref)


def test_empty_batch_is_a_no_op():
    cfg = _cfg("tiny", T=0)
    L = layer(_cfg("tiny"))
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device=DEV)
    out = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k)
    assert out.shape == (0, cfg.H)
