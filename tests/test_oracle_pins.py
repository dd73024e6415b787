"""Pins of the CPU oracle against facts fixed outside it (no GPU needed).

Each test checks the oracle against a library routine, a closed form, an
exactly constructed input, a brute-force evaluation or a hand-written case,
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule, a wrong summation order) fails
at least one of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # fp32 unit roundoff


def bits(t):
    return I.bf16_bits(t)


def torch_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by torch (round-to-nearest-even), as uint16 bits."""
    return bits(torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16))


def f32_from_bits(u):
    return np.array(u, dtype=np.uint32).view(np.float32)


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.nextafter(x, np.float32(np.inf)) - x


# --------------------------------------------------------------------------
# number format
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_rne():
    """fp32 -> bf16 rounding equals torch's round-to-nearest-even conversion."""
    rng = np.random.default_rng(0)
    raw = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001,
                        0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F807FFF, 0x7F7F8000,
                        0x7F7F7FFF, 0x807FFFFF, 0x00008000, 0x00018000], dtype=np.uint32)
    v = np.concatenate([raw, special]).view(np.float32)
    ours = O.f32_to_bf16(v)
    ref = torch_bf16_bits(v)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays NaN (exponent all ones, mantissa nonzero)
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


# --------------------------------------------------------------------------
# D1 router logits
# --------------------------------------------------------------------------

@pytest.mark.parametrize("H", [64, 256, 960, 2048])
def test_logits_equal_chunked_sequential_fp32_sum(H):
    """Logits: ascending fp32 running sums over 256-wide chunks of i, then an
    ascending fp32 running sum of the chunk sums.

    numpy's cumulative sum in float32 adds left to right with one rounding per
    step; bf16 x bf16 products are exact in fp32.  H = 960 has a short last
    chunk.
    """
    cfg = I.scaled(I.CONFIGS["mid"], T=6, H=H, E=16)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    got = O.router_logits(bits(x), bits(L["w_router"]))
    xf = x.float().numpy()
    wf = L["w_router"].float().numpy()
    for t in range(cfg.T):
        for e in range(cfg.E):
            prod = (xf[t] * wf[e]).astype(np.float32)
            assert np.array_equal(prod.astype(np.float64), xf[t].astype(np.float64) * wf[e])
            parts = [np.cumsum(prod[c:c + 256], dtype=np.float32)[-1] for c in range(0, H, 256)]
            ref = np.cumsum(np.array(parts, dtype=np.float32), dtype=np.float32)[-1]
            assert got[t, e].view(np.uint32) == np.float32(ref).view(np.uint32), (t, e)
    # the order is not arbitrary: a single running sum differs somewhere
    if H > 256:
        single = np.array([[np.cumsum((xf[t] * wf[e]).astype(np.float32), dtype=np.float32)[-1]
                            for e in range(cfg.E)] for t in range(cfg.T)], dtype=np.float32)
        assert not np.array_equal(single.view(np.uint32), got.view(np.uint32))


def test_logits_within_recursive_summation_bound():
    """|l - exact| <= gamma_H * sum|x_i w_i| (recursive summation error bound)."""
    cfg = I.scaled(I.CONFIGS["large"], T=16, H=6144, E=32)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    got = O.router_logits(bits(x), bits(L["w_router"])).astype(np.float64)
    xd = x.double().numpy()
    wd = L["w_router"].double().numpy()
    exact = xd @ wd.T                       # products exact in fp64; fp64 sum error ~1e-16
    absum = np.abs(xd) @ np.abs(wd).T
    n = cfg.H
    gamma = n * U / (1 - n * U)
    assert np.all(np.abs(got - exact) <= gamma * absum + 1e-12 * absum)
    # and not trivially: the fp32 chain does differ from the exact value somewhere
    assert np.any(got != exact)


def test_logits_exact_by_construction_on_tie_inputs():
    """Constructed stress tokens have logits equal to their target z bitwise."""
    cfg = I.scaled(I.CONFIGS["tie"], T=64)
    d = I.make_tie_inputs(cfg)
    got = O.router_logits(bits(d["x"]), bits(d["w_router"]))
    stress = np.nonzero(d["kind"] >= 2)[0]
    assert np.array_equal(got[stress].view(np.uint32), d["z"][stress].view(np.uint32))


# --------------------------------------------------------------------------
# D3 top-k
# --------------------------------------------------------------------------

def _parse_key(s):
    s = s.strip()
    if s.startswith("0x"):
        return f32_from_bits([int(s, 16)])[0]
    return np.float32(float(s))


def load_tie_cases():
    cases = []
    with open(os.path.join(GOLDEN, "topk_ties.txt")) as f:
        for line in f:
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            name, k, keys, ids = [p.strip() for p in line.split("|")]
            cases.append((name, int(k), np.array([_parse_key(v) for v in keys.split(",")],
                                                 dtype=np.float32),
                          [int(v) for v in ids.split(",")]))
    return cases


@pytest.mark.parametrize("case", load_tie_cases(), ids=lambda c: c[0])
def test_topk_hand_built_cases(case):
    name, k, keys, expect = case
    got = O.topk_keys(keys[None, :], k)[0].tolist()
    assert got == expect, (name, keys, got, expect)


def test_topk_equals_library_sort_random():
    """Without NaN the selection is the first k of Python's sort by (-key, index)."""
    rng = np.random.default_rng(3)
    for E, k in [(8, 2), (64, 8), (256, 8), (128, 16), (16, 16), (5, 1)]:
        keys = rng.standard_normal((200, E)).astype(np.float32)
        # force many exact ties by coarse quantisation on half the rows
        keys[::2] = np.round(keys[::2] * 2) / 2
        got = O.topk_keys(keys, k)
        for r in range(keys.shape[0]):
            ref = sorted(range(E), key=lambda e: (-float(keys[r, e]), e))[:k]
            assert got[r].tolist() == ref


def test_topk_on_tie_inputs_matches_rule():
    """Routing of constructed ties and 1-ulp gaps follows the tie rule exactly."""
    cfg = I.scaled(I.CONFIGS["tie"], T=256)
    d = I.make_tie_inputs(cfg)
    ids, w, gap = O.route(bits(d["x"]), bits(d["w_router"]), cfg.k, O.SOFTMAX, True)
    for t in np.nonzero(d["kind"] >= 2)[0]:
        z = d["z"][t]
        ref = sorted(range(cfg.E), key=lambda e: (-float(z[e]), e))[:cfg.k]
        assert ids[t].tolist() == ref
        if d["kind"][t] == 2:
            assert gap[t] == 0.0
        else:
            kth = z[ref[-1]]
            assert gap[t] == float(kth) - float(np.nextafter(kth, np.float32(-np.inf)))


# --------------------------------------------------------------------------
# D2 + D4 scores and weights
# --------------------------------------------------------------------------

def test_softmax_weights_against_fp64_library():
    from scipy.special import softmax
    cfg = I.scaled(I.CONFIGS["mid"], T=64, H=512)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    ids, w, gap = O.route(bits(x), bits(L["w_router"]), cfg.k, O.SOFTMAX, renorm=False)
    l = O.router_logits(bits(x), bits(L["w_router"])).astype(np.float64)
    p = softmax(l, axis=1)
    ref = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.all(np.abs(w - ref) <= ulp32(ref))
    # the selection is the top-k of the logits (softmax is increasing)
    for t in range(cfg.T):
        assert ids[t].tolist() == sorted(range(cfg.E), key=lambda e: (-l[t, e], e))[:cfg.k]
    # renormalised: weights sum to one within k roundings
    ids2, w2, _ = O.route(bits(x), bits(L["w_router"]), cfg.k, O.SOFTMAX, renorm=True)
    assert np.array_equal(ids, ids2)
    s = w2.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= cfg.k * U * 2)
    ref2 = ref / ref.sum(axis=1, keepdims=True)
    assert np.all(np.abs(w2 - ref2) <= ulp32(ref2))


def test_sigmoid_keys_weights_and_bias_role():
    from scipy.special import expit
    cfg = I.scaled(I.CONFIGS["large"], T=64, H=512, E=32)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    b = L["bias"].numpy()
    ids, w, gap = O.route(bits(x), bits(L["w_router"]), cfg.k, O.SIGMOID, True, bias=b)
    l = O.router_logits(bits(x), bits(L["w_router"])).astype(np.float64)
    key = expit(l) + b.astype(np.float64)
    for t in range(cfg.T):
        ref = sorted(range(cfg.E), key=lambda e: (-key[t, e], e))[:cfg.k]
        # keys are taken in fp32 (a few ulp from fp64); only near-ties may differ
        if gap[t] > 1e-6:
            assert ids[t].tolist() == ref
    p = np.take_along_axis(expit(l), ids.astype(np.int64), axis=1)   # bias not in weights
    ref_w = p / p.sum(axis=1, keepdims=True)
    assert np.all(np.abs(w - ref_w) <= ulp32(ref_w))
    # the bias changes the selection
    ids0, _, _ = O.route(bits(x), bits(L["w_router"]), cfg.k, O.SIGMOID, True, bias=None)
    assert not np.array_equal(ids0, ids)


def test_special_weight_cases():
    cfg = I.scaled(I.CONFIGS["tiny"], T=16, E=1, k=1)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    ids, w, gap = O.route(bits(x), bits(L["w_router"]), 1, O.SOFTMAX, False)
    assert np.all(ids == 0) and np.all(w == 1.0)       # exp(0)/1
    assert np.all(np.isinf(gap))
    cfg2 = I.scaled(I.CONFIGS["tiny"], T=16, k=1)
    L2 = I.make_layer(cfg2)
    _, w2, _ = O.route(bits(x), bits(L2["w_router"]), 1, O.SOFTMAX, True)
    assert np.all(w2 == 1.0)                            # p / p
    # sigmoid(0) = 0.5 exactly: zero router rows
    zr = torch.zeros((4, cfg.H), dtype=torch.bfloat16)
    _, w3, _ = O.route(bits(x), bits(zr), 2, O.SIGMOID, False)
    assert np.all(w3 == 0.5)


# --------------------------------------------------------------------------
# D5 permutation
# --------------------------------------------------------------------------

def test_permutation_equals_stable_argsort():
    rng = np.random.default_rng(5)
    for T, E, k in [(64, 8, 2), (1000, 64, 8), (1, 256, 8), (333, 7, 3)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        # skew: many tokens on expert 0 when it is in their set
        counts, offsets, perm, inv = O.permute(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(perm, np.argsort(flat, kind="stable").astype(np.int32))
        assert np.array_equal(counts, np.bincount(flat, minlength=E).astype(np.int32))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
        assert offsets[-1] == T * k
        assert np.array_equal(inv[perm], np.arange(T * k, dtype=np.int32))


def test_permutation_empty_and_single_expert():
    counts, offsets, perm, inv = O.permute(np.zeros((0, 2), np.int32), 4)
    assert counts.tolist() == [0, 0, 0, 0] and offsets.tolist() == [0, 0, 0, 0, 0]
    ids = np.zeros((5, 1), np.int32)
    counts, offsets, perm, inv = O.permute(ids, 1)
    assert perm.tolist() == [0, 1, 2, 3, 4]


# --------------------------------------------------------------------------
# D6 expert FFN
# --------------------------------------------------------------------------

def test_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1: the layer is one dense SwiGLU MLP; compare with torch fp64."""
    cfg = I.scaled(I.CONFIGS["tiny"], T=32, E=1, k=1)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    r = O.forward(bits(x), bits(L["w_router"]), bits(L["w_gate"]), bits(L["w_up"]),
                  bits(L["w_down"]), 1, O.SOFTMAX, True)
    xd = x.double()
    g = xd @ L["w_gate"][0].double().T
    u = xd @ L["w_up"][0].double().T
    act = (torch.nn.functional.silu(g) * u).float().to(torch.bfloat16)   # fp64->fp32->bf16
    y = act.double() @ L["w_down"][0].double().T
    y32 = y.float().numpy()
    _, act_o = O.expert_ffn(np.arange(cfg.T), np.zeros(cfg.T), bits(x), bits(L["w_gate"]),
                            bits(L["w_up"]), bits(L["w_down"]), want_act=True)
    # act codes agree except where the two fp64 sums round to different fp32 values
    assert np.mean(act_o == bits(act)) > 0.999
    assert np.max(np.abs(r["y"] - y32)) <= 1e-6 * np.max(np.abs(y32)) + 1e-9
    # w = 1 exactly, so out = bf16(Y)
    assert np.array_equal(r["out"], torch_bf16_bits(r["y"]))


def test_transposed_weights_are_caught():
    """A transposed gate matrix gives a different result (the pin above would fail)."""
    cfg = I.scaled(I.CONFIGS["tiny"], T=4, E=1, k=1, H=256, F=256)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    y1 = O.expert_ffn(np.arange(4), np.zeros(4), bits(x), bits(L["w_gate"]), bits(L["w_up"]),
                      bits(L["w_down"]))
    wgT = L["w_gate"].transpose(1, 2).contiguous()
    y2 = O.expert_ffn(np.arange(4), np.zeros(4), bits(x), bits(wgT), bits(L["w_up"]),
                      bits(L["w_down"]))
    assert np.max(np.abs(y1 - y2)) > 1e-3 * np.max(np.abs(y1))


def test_permuted_path_equals_brute_force_dense():
    """Forward via permutation equals evaluating each (token, expert) pair directly."""
    cfg = I.CONFIGS["tiny"]
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    args = (bits(L["w_router"]), bits(L["w_gate"]), bits(L["w_up"]), bits(L["w_down"]))
    r = O.forward(bits(x), *args, cfg.k, cfg.score, cfg.renorm)
    # all E experts for every token, no permutation
    T, E = cfg.T, cfg.E
    tok = np.repeat(np.arange(T), E)
    exp_ = np.tile(np.arange(E), T)
    ydense = O.expert_ffn(tok, exp_, bits(x), *args[1:]).reshape(T, E, cfg.H)
    ysel = np.stack([ydense[t, r["ids"][t]] for t in range(T)]).reshape(T * cfg.k, cfg.H)
    assert np.array_equal(ysel.view(np.uint32), r["y"].view(np.uint32))
    out = O.combine(ysel, r["w"], T, cfg.H, cfg.k)
    assert np.array_equal(out, r["out"])
    # per-token path gives the same bits
    out2, ids2, w2, gap2 = O.forward_tokens(np.arange(T), bits(x), *args, cfg.k, cfg.score,
                                            cfg.renorm)
    assert np.array_equal(out2, r["out"]) and np.array_equal(ids2, r["ids"])
    assert np.array_equal(w2.view(np.uint32), r["w"].view(np.uint32))


def test_expert_error_within_bound():
    """Y against an exact fp64 evaluation: within fp64-level error plus one fp32 rounding."""
    cfg = I.scaled(I.CONFIGS["mid"], T=4, H=1024, F=512, E=4, k=2)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    y, act = O.expert_ffn(np.arange(4), np.array([0, 1, 2, 3]), bits(x), bits(L["w_gate"]),
                          bits(L["w_up"]), bits(L["w_down"]), want_act=True)
    a = O.bf16_to_f32(act).astype(np.float64)
    for r in range(4):
        wd = L["w_down"][r].double().numpy()
        exact = wd @ a[r]
        bound = np.abs(wd) @ np.abs(a[r]) * (cfg.F * 2.0 ** -53 * 2) + np.abs(exact) * U
        assert np.all(np.abs(y[r] - exact) <= bound + 1e-30)


def test_down_step_alone_matches_full_ffn():
    """Down projection on the FFN's own act codes reproduces the FFN's y bitwise,
    and equals a torch fp64 matmul of those codes within one fp32 rounding."""
    cfg = I.scaled(I.CONFIGS["tiny"], T=6, E=3, k=1)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    experts = np.array([0, 1, 2, 2, 1, 0])
    y, act = O.expert_ffn(np.arange(6), experts, bits(x), bits(L["w_gate"]), bits(L["w_up"]),
                          bits(L["w_down"]), want_act=True)
    y2 = O.expert_down(experts, act, bits(L["w_down"]))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    a = torch.from_numpy(O.bf16_to_f32(act).astype(np.float64))
    for r in range(6):
        ref = (L["w_down"][experts[r]].double() @ a[r]).numpy()
        assert np.all(np.abs(y2[r] - ref) <= np.abs(ref) * U + 1e-12)


# --------------------------------------------------------------------------
# D7 combine
# --------------------------------------------------------------------------

def _round_f32_exact(q: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 of an exact rational."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_combine_is_fma_chain_in_slot_order():
    """Each step is one correctly rounded w*y + acc (exact rational reference)."""
    rng = np.random.default_rng(9)
    T, H, k = 3, 64, 8
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    out = O.combine(y, w, T, H, k)
    for t in range(T):
        for h in range(H):
            acc = np.float32(0.0)
            for j in range(k):
                acc = _round_f32_exact(Fraction(float(w[t, j])) * Fraction(float(y[t * k + j, h]))
                                       + Fraction(float(acc)))
            assert out[t, h] == torch_bf16_bits(np.array([acc]))[0]


def test_combine_uses_single_rounding_fma():
    """acc = fma(w, y, acc) keeps the product's rounding error; mul-then-add loses it.

    Slot 0 loads acc = -fp32(P); slot 1 adds P = w1*y1 (inexact in fp32), so a
    fused step leaves the exact residual P - fp32(P) (nonzero, representable)
    while a separate multiply and add gives 0.
    """
    w1, y1 = np.float32(1.0 + 2.0 ** -12), np.float32(1.0 + 2.0 ** -13)
    P = Fraction(float(w1)) * Fraction(float(y1))
    p32 = _round_f32_exact(P)
    resid = P - Fraction(float(p32))
    assert resid != 0
    y = np.array([[-p32], [y1]], dtype=np.float32)
    w = np.array([[1.0, w1]], dtype=np.float32)
    got = O.bf16_to_f32(O.combine(y, w, 1, 1, 2))[0, 0]
    assert got == O.bf16_to_f32(torch_bf16_bits(np.array([float(resid)], np.float32)))[0]
    assert got != 0.0


def test_combine_order_matters_and_is_pinned():
    """A case where slot order changes the fp32 sum: the oracle follows slot order."""
    T, H, k = 1, 1, 3
    y = np.array([[1.0], [2.0 ** 24], [-(2.0 ** 24)]], dtype=np.float32)
    w = np.ones((1, 3), np.float32)
    # slot order: ((0 + 1) + 2^24) - 2^24 = 0 (1 is lost); reversed it would be 1
    assert O.bf16_to_f32(O.combine(y, w, T, H, k))[0, 0] == 0.0
    y2 = y[::-1].copy()
    assert O.bf16_to_f32(O.combine(y2, w, T, H, k))[0, 0] == 1.0


def test_combine_k1_and_dyadic_exact():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((10, 32)).astype(np.float32)
    out = O.combine(y, np.ones((10, 1), np.float32), 10, 32, 1)
    assert np.array_equal(out, torch_bf16_bits(y))
    # dyadic values: every partial sum exact, result = bf16 of the exact sum
    yd = (rng.integers(-64, 64, size=(4 * 8, 16)) / 16.0).astype(np.float32)
    wd = (rng.integers(0, 16, size=(4, 8)) / 16.0).astype(np.float32)
    out = O.combine(yd, wd, 4, 16, 8)
    exact = (wd.astype(np.float64)[:, :, None] * yd.reshape(4, 8, 16)).sum(axis=1)
    assert np.array_equal(out, torch_bf16_bits(exact.astype(np.float32)))


# --------------------------------------------------------------------------
# invariance of the definition itself
# --------------------------------------------------------------------------

def test_oracle_batch_and_thread_invariance():
    cfg = I.scaled(I.CONFIGS["tiny"], T=24)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    args = (bits(L["w_router"]), bits(L["w_gate"]), bits(L["w_up"]), bits(L["w_down"]))
    full = O.forward(bits(x), *args, cfg.k, cfg.score, cfg.renorm, nthreads=1)
    full4 = O.forward(bits(x), *args, cfg.k, cfg.score, cfg.renorm, nthreads=4)
    assert np.array_equal(full["out"], full4["out"])
    for t in (0, 7, 23):
        one = O.forward(bits(x[t:t + 1]), *args, cfg.k, cfg.score, cfg.renorm)
        assert np.array_equal(one["out"][0], full["out"][t])
        assert np.array_equal(one["ids"][0], full["ids"][t])
