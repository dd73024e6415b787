"""Pins of the oracle's downstream measurement of a decode step (no GPU).

The LM-head logits, the fp32 log-softmax and Schulman's k3 estimator are
checked against numpy's ordered sums, fp64 library routines within derived
error bounds, closed forms and hand-built cases.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special as sps
import torch

from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

U = 2.0 ** -24


def bits(t):
    return I.bf16_bits(t)


def _bf16_rows(n, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((n, d), generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("H,V", [(256, 37), (320, 300), (1024, 129)])
def test_lm_head_logits_are_the_chunked_fp32_chain(H, V):
    """z[t,v]: 256-wide chunks of h, each an ascending fp32 running sum from
    +0, chunk sums added in ascending order (numpy float32 cumsum adds left to
    right with one rounding per step; bf16 x bf16 products are exact)."""
    h = _bf16_rows(3, H, 1)
    p = _bf16_rows(V, H, 2, 0.05)
    z = O.lm_head_logits(bits(h), bits(p))
    hf, pf = h.float().numpy(), p.float().numpy()
    for t in range(3):
        for v in range(V):
            prod = (hf[t] * pf[v]).astype(np.float32)
            parts = [np.cumsum(prod[c:c + 256], dtype=np.float32)[-1] for c in range(0, H, 256)]
            ref = np.cumsum(np.array(parts, dtype=np.float32), dtype=np.float32)[-1]
            assert z[t, v].view(np.uint32) == np.float32(ref).view(np.uint32), (t, v)


def test_lm_head_logits_exact_on_dyadic_rows():
    """Rows of small integers times powers of two: every partial sum is exact,
    so z equals the exact integer dot product whatever the order."""
    rng = np.random.default_rng(3)
    H, V = 768, 50
    h = rng.integers(-8, 9, size=(2, H)).astype(np.float32)
    p = (rng.integers(-8, 9, size=(V, H)) * 0.25).astype(np.float32)
    z = O.lm_head_logits(bits(torch.from_numpy(h).to(torch.bfloat16)),
                         bits(torch.from_numpy(p).to(torch.bfloat16)))
    assert np.array_equal(z.astype(np.float64), h.astype(np.float64) @ p.astype(np.float64).T)


def _ls_bound(z, logp, chunk=256):
    """First-order bound of |fp32 log-softmax - exact|: the positive chunked sum
    S of exp(z - m) has relative error <= (chunk - 1 + nchunks + 2) u (the
    additions plus the error of expf on each term); logf, the add of m and the
    final subtraction each add half an ulp of their result."""
    V = z.shape[-1]
    nch = (V + chunk - 1) // chunk
    m = z.max(axis=-1, keepdims=True).astype(np.float64)
    lnS = sps.logsumexp(z.astype(np.float64) - m, axis=-1, keepdims=True)
    rel = (min(chunk, V) - 1 + nch + 2) * U
    return rel + U * (np.abs(lnS) + np.abs(m + lnS) + np.abs(logp.astype(np.float64))) + 1e-12


@pytest.mark.parametrize("V", [1, 7, 256, 1000, 4096, 65536])
def test_log_softmax_within_fp64_library_bound(V):
    rng = np.random.default_rng(V)
    z = (rng.standard_normal((4, V)) * 3).astype(np.float32)
    z[1] *= 10.0            # a peaked row
    logp = O.log_softmax(z)
    exact = z.astype(np.float64) - sps.logsumexp(z.astype(np.float64), axis=-1, keepdims=True)
    err = np.abs(logp.astype(np.float64) - exact)
    bound = _ls_bound(z, logp)
    assert np.all(err <= bound), float((err / bound).max())
    # normalised within the same bound
    tot = np.exp(logp.astype(np.float64)).sum(axis=-1)
    assert np.all(np.abs(tot - 1.0) <= bound.max(axis=-1) * 1.01 + 2 * V * U)


def test_log_softmax_constant_row_and_shift():
    V = 1000
    z = np.zeros((2, V), dtype=np.float32)
    z[1] += np.float32(5.0)
    logp = O.log_softmax(z)
    # exp(0) = 1 exactly, S = V exactly, so logp = -(logf(V)) (to the rounding
    # of m + logf(V) for the shifted row)
    ref = np.float32(-math.log(V))
    assert np.all(np.abs(logp[0] - ref) <= np.abs(np.spacing(ref)))
    assert np.all(np.abs(logp[1] - ref) <= 2 * np.abs(np.spacing(np.float32(5.0 + math.log(V)))))


def test_log_softmax_sum_order_is_chunked():
    """The sum of exp is taken in 256-wide chunks: a row built so that the
    chunked and the single running sum differ gives the chunked result."""
    V = 512
    # one term of 1, then terms of ~1e-8: each is lost when added to 1 (below
    # half an ulp of 1) but 256 of them summed on their own are not
    z = np.full((1, V), np.float32(math.log(1e-8)), dtype=np.float32)
    z[0, 0] = 0.0
    logp = O.log_softmax(z)
    t = np.float32(math.exp(float(z[0, 1])))
    # single running sum: 1 + tiny rounds back to 1 every step
    s_single = np.float32(1.0)
    for _ in range(V - 1):
        s_single = np.float32(s_single + t)
    # chunked: chunk 0 = 1 (+ 255 small terms, each lost), chunk 1 = 256 of them
    c1 = np.cumsum(np.full(256, t, dtype=np.float32), dtype=np.float32)[-1]
    s_chunk = np.float32(np.float32(1.0) + c1)
    assert s_single != s_chunk
    got_S = np.exp(-np.float64(logp[0, 0]))   # logp_0 = -log S
    assert abs(got_S - float(s_chunk)) < abs(got_S - float(s_single))


def test_log_softmax_chunks_are_added_in_ascending_order():
    """Chunk sums 1, t, t with t about 0.7 ulp of 1: added in ascending chunk
    order S = (1 + t) + t = 1 + 2 ulp, in descending order (t + t) + 1 =
    1 + 1 ulp."""
    V = 768
    ulp = 2.0 ** -23
    z = np.full((1, V), -np.inf, dtype=np.float32)
    z[0, 0] = 0.0
    z[0, 256] = z[0, 512] = np.float32(math.log(0.7 * ulp))
    logp = O.log_softmax(z)
    asc = -math.log(1.0 + 2 * ulp)
    desc = -math.log(1.0 + ulp)
    assert abs(float(logp[0, 0]) - asc) < abs(float(logp[0, 0]) - desc)


def _rows(seed, V, scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((3, V)) * scale).astype(np.float32)


@pytest.mark.parametrize("V", [2, 300, 65536])
def test_k3_mean_is_generalized_kl_divergence(V):
    """sum_v p_test (r - 1 - ln r) with r = p_ref / p_test equals
    sum_v [p_test ln(p_test/p_ref) - p_test + p_ref], which scipy.special.kl_div
    evaluates elementwise (a library routine)."""
    ref = O.log_softmax(_rows(1, V, 2.0))
    test = O.log_softmax(_rows(2, V, 2.0))
    mean, gk3, g = O.k3(ref, test)
    pr, pt = np.exp(ref.astype(np.float64)), np.exp(test.astype(np.float64))
    lib = sps.kl_div(pt, pr).sum(axis=-1)
    assert np.allclose(mean, lib, rtol=1e-9, atol=1e-15)
    assert np.all(mean > 0)
    # greedy token and its term
    for t in range(3):
        v = int(np.argmax(test[t]))
        assert g[t] == v
        r = pr[t, v] / pt[t, v]
        assert math.isclose(gk3[t], (r - 1) - math.log(r), rel_tol=1e-9, abs_tol=1e-15)


def test_k3_identical_is_exactly_zero_and_two_point_closed_form():
    lp = O.log_softmax(_rows(5, 4096, 3.0))
    mean, gk3, _ = O.k3(lp, lp)
    assert np.all(mean == 0.0) and np.all(gk3 == 0.0)
    # two outcomes: KL(Bern(a) || Bern(b))
    a, b = 0.3, 0.6
    test = np.log(np.array([[a, 1 - a]], dtype=np.float32))
    ref = np.log(np.array([[b, 1 - b]], dtype=np.float32))
    mean, _, g = O.k3(ref, test)
    pa, pb = np.exp(test.astype(np.float64))[0], np.exp(ref.astype(np.float64))[0]
    kl = pa[0] * math.log(pa[0] / pb[0]) + pa[1] * math.log(pa[1] / pb[1]) - pa.sum() + pb.sum()
    assert math.isclose(mean[0], kl, rel_tol=1e-12)
    assert g[0] == 1


def test_k3_greedy_tie_takes_lowest_index():
    test = np.log(np.array([[0.1, 0.4, 0.1, 0.4]], dtype=np.float32))
    ref = np.log(np.array([[0.25, 0.25, 0.25, 0.25]], dtype=np.float32))
    _, _, g = O.k3(ref, test)
    assert g[0] == 1


def test_k3_near_identical_rows_against_the_series():
    """Rows a few ulps apart: each term expm1(d) - d equals the series
    d^2/2 + d^3/6 + d^4/24 to fp64 precision (|d| < 1e-5), which an
    evaluation as exp(d) - 1 - d would miss by cancellation."""
    test = O.log_softmax(_rows(3, 4096, 1.0))
    rng = np.random.default_rng(6)
    ref = (test.astype(np.float64) * (1.0 + rng.uniform(-3e-7, 3e-7, test.shape))).astype(np.float32)
    mean, gk3, g = O.k3(ref, test)
    d = ref.astype(np.float64) - test.astype(np.float64)
    assert np.abs(d).max() < 1e-5 and np.any(d != 0)
    series = d * d / 2 + d ** 3 / 6 + d ** 4 / 24
    lib = (np.exp(test.astype(np.float64)) * series).sum(axis=-1)
    assert np.allclose(mean, lib, rtol=1e-9, atol=0)
    for t in range(3):
        assert math.isclose(gk3[t], series[t, g[t]], rel_tol=1e-9, abs_tol=1e-300)


# ---------------------------------------------------------------------------
# The log-softmax's transcendentals and sums, pinned to the last bit.
# ---------------------------------------------------------------------------

def _cr_f32(d):
    """Round a high-precision Decimal to the nearest fp32, ties to even (written
    out here from the IEEE definition: the nearest of the fp32 neighbours of
    the double nearest d, compared in Decimal arithmetic)."""
    from decimal import Decimal
    f = np.float32(float(d))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Decimal(float(c)) - d), int(c.view(np.uint32)) & 1))


def test_exp32_and_log32_are_correctly_rounded():
    """exp32 / log32 equal the exact exponential and logarithm (Python's
    decimal module at 60 digits, which rounds them correctly at its precision)
    rounded to the nearest fp32, on arguments the log-softmax meets: z - m in
    [-110, 0] (down to subnormal and zero results) and sums in [1, 2^17]."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    rng = np.random.default_rng(12)
    a = np.concatenate([-rng.exponential(4.0, 3000), -rng.uniform(80, 110, 300),
                        [0.0, -1e-30, -2.0 ** -24, -87.3, -103.9, -150.0]]).astype(np.float32)
    for v in a:
        want = _cr_f32(Decimal(float(v)).exp())
        got = O.exp32(v)
        assert got.view(np.uint32) == want.view(np.uint32), (float(v), float(got), float(want))
    s = np.concatenate([rng.uniform(1.0, 2.0 ** 17, 3000), [1.0, 1.0 + 2 ** -23, 65536.0]])
    for v in s.astype(np.float32):
        want = _cr_f32(Decimal(float(v)).ln())
        got = O.log32(v)
        assert got.view(np.uint32) == want.view(np.uint32), (float(v), float(got), float(want))
    assert O.exp32(-np.inf) == 0.0 and O.exp32(0.0) == 1.0 and O.log32(1.0) == 0.0


def test_log_softmax_sums_in_fp32_from_the_first_term():
    """A chunk of one term 1 (z = m) followed by 255 terms t < 2^-24 (half an
    fp32 ulp of 1): in the fp32 chain each t is lost, S = 1 exactly, log 1 = 0
    and logp = z exactly.  An fp64 (or compensated, or pairwise) sum keeps the
    255 t and moves logp_0 by about -2.5e-6."""
    V = 256
    z = np.full((1, V), np.float32(-18.5), dtype=np.float32)   # exp(-18.5) ~ 9.2e-9
    z[0, 0] = 0.0
    logp = O.log_softmax(z)
    assert logp[0, 0] == 0.0
    assert np.array_equal(logp[0, 1:], z[0, 1:])


def test_log_softmax_chain_runs_in_ascending_v():
    """The same terms with the 1 last: the ascending chain first adds the 255
    terms t (about 255 t = 2.4e-6 in all), which then survive the add of 1, so
    logp at the maximum is -log(1 + ~255 t) instead of 0 (descending order would
    lose them)."""
    V = 256
    z = np.full((1, V), np.float32(-18.5), dtype=np.float32)
    z[0, V - 1] = 0.0
    logp = O.log_softmax(z)
    t = math.exp(-18.5)
    assert logp[0, V - 1] < -2e-6
    assert abs(float(logp[0, V - 1]) + 255 * t) < 2 * 2.0 ** -23


def test_log_softmax_chunks_sum_on_their_own():
    """Two chunks: [1, t x 255] and [t x 256], t < 2^-24.  Chunk 0 sums to 1,
    chunk 1 to ~256 t, and S = 1 + 256 t: logp_0 ~ -256 t.  A single running
    fp32 sum gives 0 and an fp64 sum about -511 t; both are told apart."""
    V = 512
    z = np.full((1, V), np.float32(-18.5), dtype=np.float32)
    z[0, 0] = 0.0
    logp = O.log_softmax(z)
    t = math.exp(-18.5)
    got = -float(logp[0, 0])
    assert abs(got - 256 * t) < 2 * 2.0 ** -23          # ~2.4e-6, within 2 ulp of 1
    assert abs(got - 511 * t) > 1e-6 and got > 1e-6


def test_k3_sums_fp64_terms_in_chunks():
    """k3 terms: v = 0 gives T0 = expm1(1) - 1 (~0.718); every other v gives
    exp(-38) * T0 (~2.3e-17, below half an fp64 ulp of T0).  In one running sum
    they are all lost and the mean is T0; in the chunked order chunk 0 is T0 and
    chunk 1 sums 256 of them (~5.8e-15, ~52 ulps of T0) before it is added."""
    V = 512
    test = np.full((1, V), np.float32(-38.0), dtype=np.float32)
    test[0, 0] = 0.0
    ref = test + np.float32(1.0)                          # d = 1 exactly everywhere
    mean, _, g = O.k3(ref, test)
    T0 = math.expm1(1.0) - 1.0
    small = math.exp(-38.0) * T0
    ulp = 2.0 ** -53
    assert abs((mean[0] - T0) - 256 * small) <= 3 * ulp
    assert g[0] == 0


@pytest.mark.parametrize("m", [9.25, 1000.0, -3.5])
def test_log_softmax_final_steps_round_in_fp32(m):
    """A row of two equal logits m: both terms are exp(0) = 1, S = 2 exactly,
    so lse = fp32(m + log32(2)) and logp = fp32(m - lse), with log32(2) the
    correctly rounded fp32 log 2 (decimal module).  At m = 9.25 an fp64 add of
    m and log 2 rounds to another fp32 than the fp32 add does, and at every m
    (z - m) - log32(2) (two subtractions) differs from z - lse."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    l2 = _cr_f32(Decimal(2).ln())
    z = np.full((1, 2), np.float32(m), dtype=np.float32)
    logp = O.log_softmax(z)
    lse = np.float32(np.float32(m) + l2)
    want = np.float32(np.float32(m) - lse)
    assert logp[0, 0].view(np.uint32) == want.view(np.uint32), (float(logp[0, 0]), float(want))
    assert logp[0, 1] == logp[0, 0]


def test_k3_chunk_sums_are_added_in_ascending_order():
    """Chunk sums T0, c, c with c about 0.7 fp64 ulp of T0 (one term per later
    chunk; every other term is exp(q) * 0 = 0 since ref = test there): in
    ascending chunk order the mean is (T0 + c) + c = T0 + 2 ulp, in descending
    order T0 + (c + c) = T0 + 1 ulp."""
    V = 768
    test = np.full((1, V), np.float32(-200.0), dtype=np.float32)
    ref = test.copy()
    T0 = math.expm1(1.0) - 1.0
    ulp = 2.0 ** -53                                      # T0 in [0.5, 1)
    a = np.float32(math.log(0.7 * ulp / T0))
    test[0, 0], ref[0, 0] = 0.0, 1.0
    for v in (256, 512):
        test[0, v], ref[0, v] = a, a + np.float32(1.0)
    assert float(ref[0, 256]) - float(test[0, 256]) == 1.0
    mean, _, _ = O.k3(ref, test)
    c = math.exp(float(a)) * T0
    asc = (T0 + c) + c
    desc = T0 + (c + c)
    assert asc != desc
    assert abs(mean[0] - asc) < abs(mean[0] - desc)
