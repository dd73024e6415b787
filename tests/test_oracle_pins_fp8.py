"""Pins of the oracle's FP8 rollout path (no GPU): the e4m3 code table and
rounding against the OCP definition and torch's float8_e4m3fn, the block
exponent's closed form, and the block-scaled GEMM against an fp64 library
matmul of the dequantised codes within its fp32 accumulation bound."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from serve_router_gemm_amd import inputs as I

U = 2.0 ** -24


def bits(t):
    return I.bf16_bits(t)


def test_e4m3_code_table():
    codes = np.arange(256, dtype=np.uint8)
    got = O.e4m3_to_f32(codes)
    s = np.where(codes >= 128, -1.0, 1.0)
    ex = (codes >> 3) & 15
    m = codes & 7
    ref = np.where(ex == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (ex.astype(np.float64) - 7))
    ref = s * ref
    nan = (ex == 15) & (m == 7)
    assert np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan].astype(np.float64), ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9
    tl = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(got[~nan], tl[~nan])


def test_e4m3_rounding_matches_torch_and_round_trips():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(100000) * 1e-2,
                        rng.standard_normal(100000) * 3e-3]).astype(np.float32)
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_to_f32(codes)
    fin = ~np.isnan(vals)
    # every exact midpoint between neighbouring codes (ties to even)
    pos = np.sort(np.unique(vals[fin & (vals >= 0)]))
    mids = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, vals[fin]])
    ours = O.f32_to_e4m3(v)
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
    assert np.array_equal(O.f32_to_e4m3(vals[fin]), codes[fin])      # decode -> encode
    assert O.f32_to_e4m3(np.array([1000.0, -1e9], np.float32)).tolist() == [0x7E, 0xFE]


@pytest.mark.parametrize("k", [-20, -8, 0, 3, 12])
def test_fp8_block_exponent_closed_form(k):
    a = np.float32(448.0 * 2.0 ** k)
    assert O.fp8_block_exp(a) == k
    assert O.fp8_block_exp(np.nextafter(a, np.float32(np.inf))) == k + 1
    rng = np.random.default_rng(k + 50)
    for amax in rng.uniform(1e-6, 1e3, 200).astype(np.float32):
        e = O.fp8_block_exp(amax)
        assert 448.0 * 2.0 ** (e - 1) < amax <= 448.0 * 2.0 ** e
    assert O.fp8_block_exp(0.0) == 0


def test_quantize_blocks_are_scaled_e4m3():
    g = torch.Generator().manual_seed(1)
    w = (torch.randn((256, 384), generator=g) * 0.02).to(torch.bfloat16)
    w[5, 7] = 3.0                                # one large entry in block (0, 0)
    wb = bits(w)
    q, e = O.quantize_fp8(wb, 128)
    assert q.shape == (256, 384) and e.shape == (2, 3)
    wf = w.float().numpy()
    for rb in range(2):
        for kb in range(3):
            blk = wf[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128]
            ee = int(e[rb, kb])
            assert ee == O.fp8_block_exp(np.abs(blk).max())
            lib = torch.from_numpy(np.ldexp(blk, -ee).astype(np.float32)).to(
                torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[rb * 128:(rb + 1) * 128, kb * 128:(kb + 1) * 128], lib)
    # activation rows: one exponent per (row, 128-block)
    qa, ea = O.quantize_fp8(wb, 1)
    assert ea.shape == (256, 3)
    assert ea[5, 0] == O.fp8_block_exp(3.0)


def _block_scales(rows, cols, seed):
    """A different power of two per 128 x 128 block, so that every block has
    its own exponent and a mis-indexed exponent shows."""
    rng = np.random.default_rng(seed)
    f = 2.0 ** rng.integers(-4, 5, size=(rows // 128, cols // 128))
    return torch.from_numpy(np.repeat(np.repeat(f, 128, axis=0), 128, axis=1)).float()


def _fp8_layer(T=6, H=256, F=384, E=3, seed=2):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((T, H), generator=g) * _block_scales(128, H, seed)[0]).to(torch.bfloat16)
    wg = (torch.randn((E, F, H), generator=g) * 0.05 * _block_scales(F, H, seed + 1)).to(torch.bfloat16)
    wu = (torch.randn((E, F, H), generator=g) * 0.05 * _block_scales(F, H, seed + 2)).to(torch.bfloat16)
    wd = (torch.randn((E, H, F), generator=g) * 0.05 * _block_scales(H, F, seed + 3)).to(torch.bfloat16)
    xq, xe = O.quantize_fp8(bits(x), 1)
    wq = {}
    wq["wgq"], wq["wge"] = O.quantize_fp8(bits(wg), 128)
    wq["wuq"], wq["wue"] = O.quantize_fp8(bits(wu), 128)
    wq["wdq"], wq["wde"] = O.quantize_fp8(bits(wd), 128)
    return x, wg, wu, wd, xq, xe, wq


def _deq(q, e, block_rows):
    """Dequantised codes (fp64): q * 2^e by blocks."""
    v = O.e4m3_to_f32(q).astype(np.float64)
    er = np.repeat(np.repeat(e.astype(np.float64), block_rows, axis=-2), 128, axis=-1)
    return v * 2.0 ** er


def test_fp8_gemm_against_library_matmul_of_dequantised_codes():
    """y[h] from the oracle vs an fp64 library matmul of the dequantised act
    codes and weights: the oracle's exact block sums, scaled exactly, are
    added in fp32 over nb blocks: |y - ref| <= gamma_nb * sum_kb |block_kb|."""
    x, wg, wu, wd, xq, xe, wq = _fp8_layer()
    T, E = x.shape[0], wg.shape[0]
    toks = np.repeat(np.arange(T), E)
    exps = np.tile(np.arange(E), T)
    y, act = O.expert_ffn_fp8(toks, exps, xq, xe, wq["wgq"], wq["wge"], wq["wuq"], wq["wue"],
                              wq["wdq"], wq["wde"], want_act=True)
    aq, ae = O.quantize_fp8(act, 1)
    a_deq = _deq(aq, ae, 1)
    F = act.shape[1]
    nb = F // 128
    for i, e in enumerate(exps):
        wd_deq = _deq(wq["wdq"][e], wq["wde"][e], 128)           # [H, F]
        blocks = np.stack([a_deq[i, b * 128:(b + 1) * 128] @ wd_deq[:, b * 128:(b + 1) * 128].T
                           for b in range(nb)])                  # exact in fp64
        ref = blocks.sum(axis=0)
        gamma = nb * U / (1 - nb * U)
        assert np.all(np.abs(y[i] - ref) <= gamma * np.abs(blocks).sum(axis=0) + 1e-30)


def test_fp8_gemm_exact_on_small_integer_codes():
    """Codes that are small integers with exponent 0: every block sum and the
    fp32 accumulation are exact, so the GEMM equals the integer matmul."""
    rng = np.random.default_rng(7)
    T, H, F, E = 2, 256, 128, 1
    ints = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    wint = rng.integers(-4, 5, size=(E, H, F)).astype(np.float32)
    xq = O.f32_to_e4m3(ints)
    xe = np.zeros((T, H // 128), np.int8)
    wdq = O.f32_to_e4m3(wint)
    wde = np.zeros((E, H // 128, F // 128), np.int8)
    # gate/up chosen so that act is exactly representable: g = u = 0 gives act 0;
    # use the down GEMM alone through a one-expert layer with F = 128 codes
    act = O.f32_to_bf16(np.zeros((T, F), np.float32))
    aq, ae = O.quantize_fp8(act, 1)
    assert np.all(aq == 0) and np.all(ae == 0)
    # the block-scaled dot of integer codes: check through the gate GEMM of a
    # layer whose up weights make u = 1 exactly (act = bf16(silu(g)))
    ref = ints.astype(np.float64) @ wint[0].astype(np.float64)          # [T, F]
    assert np.all(np.abs(ref) < 2 ** 24)
    wgq = O.f32_to_e4m3(np.transpose(wint, (0, 2, 1)))                  # [E, F, H]
    wge = np.zeros((E, F // 128, H // 128), np.int8)
    ones = np.zeros((E, F, H), np.float32)
    ones[:, :, 0] = 1.0                                                 # u = x[:, 0]
    xq1 = xq.copy()
    xq1[:, 0] = O.f32_to_e4m3(np.ones(T, np.float32))                   # x[:, 0] = 1
    ref = O.e4m3_to_f32(xq1).astype(np.float64) @ wint[0].astype(np.float64)
    wuq = O.f32_to_e4m3(ones)
    y, act = O.expert_ffn_fp8(np.arange(T), np.zeros(T), xq1, xe, wgq, wge, wuq, wge,
                              np.zeros((E, H, F), np.uint8), np.zeros((E, H // 128, F // 128),
                                                                     np.int8), want_act=True)
    g = torch.from_numpy(ref)
    expect = bits((g / (1 + torch.exp(-g))).float().to(torch.bfloat16))
    assert np.array_equal(act, expect)
    assert np.all(y == 0.0)


def test_fp8_layer_close_to_bf16_layer():
    """The FP8 layer approximates the bf16 layer (same routing): e4m3 keeps 3
    mantissa bits, so outputs agree to a few percent of their scale."""
    cfg = I.scaled(I.CONFIGS["tiny"], T=16, H=256, F=384)
    L = I.make_layer(cfg)
    x = I.make_x(cfg)
    xb = bits(x)
    hb = {n: bits(L[n]) for n in ("w_router", "w_gate", "w_up", "w_down")}
    xq, xe = O.quantize_fp8(xb, 1)
    wq = {}
    wq["wgq"], wq["wge"] = O.quantize_fp8(hb["w_gate"], 128)
    wq["wuq"], wq["wue"] = O.quantize_fp8(hb["w_up"], 128)
    wq["wdq"], wq["wde"] = O.quantize_fp8(hb["w_down"], 128)
    rows = np.arange(cfg.T)
    out8, ids8, _ = O.forward_tokens_fp8(rows, xb, hb["w_router"], xq, xe, wq, cfg.k, cfg.score,
                                         cfg.renorm)
    out16, ids16, _, _ = O.forward_tokens(rows, xb, hb["w_router"], hb["w_gate"], hb["w_up"],
                                          hb["w_down"], cfg.k, cfg.score, cfg.renorm)
    assert np.array_equal(ids8, ids16)
    a = O.bf16_to_f32(out8).astype(np.float64)
    b = O.bf16_to_f32(out16).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-4 < rel < 0.1, rel


def test_fp8_block_exponent_clamp():
    """The exponent travels as a signed byte and a biased scale byte: tiny
    blocks take -127 (and still quantise to the scaled e4m3 codes), an
    infinite amax takes 127."""
    tiny = np.float32(448.0 * 2.0 ** -130)
    assert O.fp8_block_exp(tiny) == -127
    assert O.fp8_block_exp(np.float32(448.0 * 2.0 ** -127)) == -127
    assert O.fp8_block_exp(np.float32(448.0 * 2.0 ** -126)) == -126
    assert O.fp8_block_exp(np.float32(np.inf)) == 127
    assert O.fp8_block_exp(np.float32(3.0e38)) == 120           # largest finite bf16 range
    v = torch.full((1, 128), 2.0 ** -128, dtype=torch.bfloat16)
    v[0, 3] = -(2.0 ** -126)
    q, e = O.quantize_fp8(bits(v), 1)
    assert e[0, 0] == -127
    lib = torch.from_numpy(np.ldexp(v.float().numpy(), 127).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, lib)
    assert O.e4m3_to_f32(q[0, :1])[0] == 0.5 and O.e4m3_to_f32(q[0, 3:4])[0] == -2.0


def test_fp8_gemm_alone_against_library_matmul():
    """orc_fp8_gemm vs an fp64 library matmul of dequantised codes, block by
    block (each block sum exact in fp64), added in fp32 in ascending block
    order: equal bit for bit."""
    rng = np.random.default_rng(11)
    n, K, N, E = 7, 384, 256, 3
    a = (rng.standard_normal((n, K)) * rng.choice([1e-3, 1.0, 30.0], (n, 1)) *
         np.repeat(2.0 ** rng.integers(-4, 5, size=(n, K // 128)), 128, axis=1)).astype(np.float32)
    w = (rng.standard_normal((E, N, K)) * 0.02 *
         np.stack([_block_scales(N, K, 20 + e).numpy() for e in range(E)])).astype(np.float32)
    aq, ae = O.quantize_fp8(O.f32_to_bf16(a), 1)
    wq, we = O.quantize_fp8(O.f32_to_bf16(w), 128)
    assert len(np.unique(we)) > 4 and len(np.unique(ae)) > 4       # blocks differ
    experts = rng.integers(0, E, n)
    y = O.fp8_gemm(aq, ae, experts, wq, we)
    a_deq = _deq(aq, ae, 1)
    for i, e in enumerate(experts):
        w_deq = _deq(wq[e], we[e], 128)                          # [N, K]
        acc = np.zeros(N, np.float32)
        for b in range(K // 128):
            blk = a_deq[i, b * 128:(b + 1) * 128] @ w_deq[:, b * 128:(b + 1) * 128].T
            acc = (acc + blk.astype(np.float32)).astype(np.float32)
        assert np.array_equal(y[i], acc)


def test_fp8_gemm_alone_exact_on_small_integers():
    rng = np.random.default_rng(12)
    n, K, N = 5, 256, 128
    ai = rng.integers(-6, 7, (n, K)).astype(np.float32)
    wi = rng.integers(-6, 7, (1, N, K)).astype(np.float32)
    y = O.fp8_gemm(O.f32_to_e4m3(ai), np.zeros((n, 2), np.int8), np.zeros(n),
                   O.f32_to_e4m3(wi), np.zeros((1, 1, 2), np.int8))
    assert np.array_equal(y.astype(np.float64), ai.astype(np.float64) @ wi[0].T.astype(np.float64))
    # exponents scale exactly: 2^(ea + ew)
    y2 = O.fp8_gemm(O.f32_to_e4m3(ai), np.full((n, 2), 3, np.int8), np.zeros(n),
                    O.f32_to_e4m3(wi), np.full((1, 1, 2), -5, np.int8))
    assert np.array_equal(y2, y * np.float32(2.0 ** -2))


def test_fp8_ffn_gate_up_equals_the_gemm():
    """The FFN's act is bf16(silu(g) * u) of the block-scaled GEMM (pinned on
    its own above) applied to the gate and up weights, every weight block with
    its own exponent: a mis-indexed gate or up exponent shows here."""
    x, wg, wu, wd, xq, xe, wq = _fp8_layer()
    T, E = x.shape[0], wg.shape[0]
    assert len(np.unique(wq["wge"])) > 4 and len(np.unique(wq["wue"])) > 4
    toks = np.repeat(np.arange(T), E)
    exps = np.tile(np.arange(E), T)
    _, act = O.expert_ffn_fp8(toks, exps, xq, xe, wq["wgq"], wq["wge"], wq["wuq"], wq["wue"],
                              wq["wdq"], wq["wde"], want_act=True)
    g = O.fp8_gemm(xq[toks], xe[toks], exps, wq["wgq"], wq["wge"]).astype(np.float64)
    u = O.fp8_gemm(xq[toks], xe[toks], exps, wq["wuq"], wq["wue"]).astype(np.float64)
    ref = O.f32_to_bf16((g / (1.0 + np.exp(-g)) * u).astype(np.float32))
    assert np.array_equal(act, ref)
