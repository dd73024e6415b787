"""Pins of the oracle's router replay (no GPU): the weights of given experts
against numpy's fp64 softmax / sigmoid, invalid ids, and the layer with a
forced expert against a dense fp64 SwiGLU MLP."""
from __future__ import annotations

import numpy as np
import scipy.special as sps
import torch

from oracle import oracle as O
from serve_router_gemm_amd import inputs as I


def bits(t):
    return I.bf16_bits(t)


def _np_weights(logits, ids, score, renorm):
    """D4 in numpy fp64: probabilities of the given experts (0 for ids outside
    [0,E)), renormalised over the valid ones, rounded to fp32 once."""
    l = logits.astype(np.float64)
    E = l.shape[1]
    valid = (ids >= 0) & (ids < E)
    safe = np.where(valid, ids, 0)
    if score == O.SOFTMAX:
        p_all = sps.softmax(l, axis=1)
    else:
        p_all = sps.expit(l)
    p = np.take_along_axis(p_all, safe, axis=1) * valid
    if renorm:
        D = p.sum(axis=1, keepdims=True)
        p = np.divide(p, D, out=np.zeros_like(p), where=D > 0)
    return p.astype(np.float32)


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def test_replay_weights_match_fp64_library_for_routed_and_random_ids():
    for name, score in (("tiny", O.SOFTMAX), ("mid", O.SOFTMAX)):
        cfg = I.scaled(I.CONFIGS[name], T=40)
        L = I.make_layer(cfg)
        x = I.make_x(cfg)
        xb, wrb = bits(x), bits(L["w_router"])
        logits = O.router_logits(xb, wrb)
        ids, w, _ = O.route(xb, wrb, cfg.k, score, cfg.renorm)
        w_rep = O.replay_weights(xb, wrb, ids, score, cfg.renorm)
        assert np.array_equal(w_rep, w)          # the routed ids give the routed weights
        assert np.all(_ulps(w_rep, _np_weights(logits, ids, score, cfg.renorm)) <= 1)
        rng = np.random.default_rng(1)
        rid = rng.integers(0, cfg.E, size=ids.shape).astype(np.int32)
        w_r = O.replay_weights(xb, wrb, rid, score, cfg.renorm)
        assert np.all(_ulps(w_r, _np_weights(logits, rid, score, cfg.renorm)) <= 1)
    # sigmoid scores, with and without renormalisation
    cfg = I.scaled(I.CONFIGS["large"], T=8, H=256, E=32, F=128)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    xb, wrb = bits(x), bits(L["w_router"])
    logits = O.router_logits(xb, wrb)
    rid = np.random.default_rng(2).integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)
    for renorm in (True, False):
        w_r = O.replay_weights(xb, wrb, rid, O.SIGMOID, renorm)
        assert np.all(_ulps(w_r, _np_weights(logits, rid, O.SIGMOID, renorm)) <= 1)
        # softmax without renormalisation: the probability over all E experts
        w_s = O.replay_weights(xb, wrb, rid, O.SOFTMAX, renorm)
        assert np.all(_ulps(w_s, _np_weights(logits, rid, O.SOFTMAX, renorm)) <= 1)


def test_replay_invalid_ids_get_no_weight_and_no_output():
    cfg = I.scaled(I.CONFIGS["tiny"], T=12)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    xb = bits(x)
    hb = {n: bits(L[n]) for n in ("w_router", "w_gate", "w_up", "w_down")}
    logits = O.router_logits(xb, hb["w_router"])
    ids = np.random.default_rng(3).integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)
    ids[::3, 1] = -1
    ids[1::3, 0] = cfg.E + 5
    ids[2, :] = -7                                 # a token with no valid expert
    invalid = (ids < 0) | (ids >= cfg.E)
    for score, renorm in ((O.SIGMOID, True), (O.SIGMOID, False), (O.SOFTMAX, False)):
        w_s = O.replay_weights(xb, hb["w_router"], ids, score, renorm)
        assert np.all(_ulps(w_s, _np_weights(logits, ids, score, renorm)) <= 1)
        assert np.all(w_s[invalid] == 0.0)
    out, w = O.forward_replay(xb, hb["w_router"], ids, hb["w_gate"], hb["w_up"], hb["w_down"],
                              O.SOFTMAX, True)
    assert np.all(_ulps(w, _np_weights(logits, ids, O.SOFTMAX, True)) <= 1)
    assert np.all(w[invalid] == 0.0)
    assert np.all(out[2] == 0)                     # bf16 +0
    # recorded weights: an invalid id's expert output is 0 whatever its weight,
    # so the out equals that of the same weights with those slots zeroed
    wrec = np.random.default_rng(4).uniform(0.1, 1.0, size=ids.shape).astype(np.float32)
    out_rec, _ = O.forward_replay(xb, hb["w_router"], ids, hb["w_gate"], hb["w_up"],
                                  hb["w_down"], O.SOFTMAX, True, w=wrec)
    wz = np.where(invalid, np.float32(0), wrec)
    out_z, _ = O.forward_replay(xb, hb["w_router"], ids, hb["w_gate"], hb["w_up"], hb["w_down"],
                                O.SOFTMAX, True, w=wz)
    assert np.array_equal(out_rec, out_z)
    assert np.all(out_rec[2] == 0)
    # a token with one valid slot of weight 1 equals that expert alone (k = 1)
    t = 0
    j = int(np.nonzero((ids[t] >= 0) & (ids[t] < cfg.E))[0][0])
    if np.count_nonzero((ids[t] >= 0) & (ids[t] < cfg.E)) == 1:
        one, _ = O.forward_replay(xb[t:t + 1], hb["w_router"], ids[t:t + 1, j:j + 1],
                                  hb["w_gate"], hb["w_up"], hb["w_down"], O.SOFTMAX, True)
        assert np.array_equal(out[t], one[0])


def test_replay_forced_expert_is_dense_swiglu_mlp():
    """k = 1 replayed onto expert e with weight 1: the layer is that expert's
    dense SwiGLU MLP (torch fp64), rounded once to bf16."""
    cfg = I.scaled(I.CONFIGS["tiny"], T=24, k=1)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    e = 5
    ids = np.full((cfg.T, 1), e, dtype=np.int32)
    out, w = O.forward_replay(bits(x), bits(L["w_router"]), ids, bits(L["w_gate"]),
                              bits(L["w_up"]), bits(L["w_down"]), O.SOFTMAX, True)
    assert np.all(w == 1.0)
    xd = x.double()
    g = xd @ L["w_gate"][e].double().T
    u = xd @ L["w_up"][e].double().T
    act = (torch.nn.functional.silu(g) * u).float().to(torch.bfloat16)
    y = (act.double() @ L["w_down"][e].double().T).float()
    ref = bits(y.to(torch.bfloat16))
    # equal except where the act codes (fp64 sums rounded to fp32) differ
    assert np.mean(out == ref) > 0.99
    of = (out.astype(np.uint32) << 16).view(np.float32)
    rf = (ref.astype(np.uint32) << 16).view(np.float32)
    assert np.max(np.abs(of - rf)) <= 2e-2 + 1e-2 * np.max(np.abs(rf))
    # recorded weights are used as given
    w2 = np.full((cfg.T, 1), 0.5, dtype=np.float32)
    half, wu = O.forward_replay(bits(x), None, ids, bits(L["w_gate"]), bits(L["w_up"]),
                                bits(L["w_down"]), O.SOFTMAX, True, w=w2)
    assert np.array_equal(wu, w2)
    hf = (half.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(hf, (bits(torch.from_numpy(0.5 * of).to(torch.bfloat16))
                               .astype(np.uint32) << 16).view(np.float32))
