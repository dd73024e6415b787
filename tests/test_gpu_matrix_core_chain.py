"""The router's fp32 chains on the matrix cores.

Router logits (and the decode step's vocabulary projection) are sums taken in
one pinned order: 256-wide chunks, each an ascending fp32 fused multiply-add
chain from +0, chunk sums added in ascending order (Fireworks page
"位级一致：前沿训练的差异化关键", section "为什么比特级一致是一个复杂的问题": a
fixed reduction order for the router).  The library takes those chains on the
VALU for few tokens and on the matrix cores (v_mfma_f32_32x32x1_2b_f32, one
product added per instruction) for larger batches.  The two are the same
chain only if the instruction's add rounds as the VALU's fused multiply-add
does on every fp32 class; these rows make the classes occur: products that
underflow to denormals or to zero, denormal running sums, products that
overflow, exact cancellation to signed zeros, infinities and NaN."""
from __future__ import annotations

import numpy as np
import torch

from helpers import DEV, bits, gpu, log
from oracle import oracle as O
from serve_router_gemm_amd import moe as M

pytestmark = gpu


def _bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 values that are bf16-representable -> bf16 tensor (exact)."""
    u = a.astype(np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return torch.from_numpy((u >> 16).astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def _rows(rng, n, H, family):
    """n rows of H bf16-representable fp32 values of one family."""
    m = (rng.standard_normal((n, H)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    if family == "normal":
        return m
    if family == "tiny":        # products near and below the fp32 denormal range
        return np.ldexp(m, rng.integers(-75, -55, size=(n, H))).astype(np.float32)
    if family == "huge":        # products that overflow to +-inf
        return np.ldexp(m, rng.integers(55, 70, size=(n, H))).astype(np.float32)
    if family == "cancel":      # equal and opposite pairs: sums that return to zero
        r = m.copy()
        r[:, 1::2] = -r[:, 0::2]
        return r
    if family == "zeros":       # signed zeros among small values
        r = np.ldexp(m, -70).astype(np.float32)
        z = rng.random((n, H)) < 0.5
        r[z] = np.where(rng.random(int(z.sum())) < 0.5, -0.0, 0.0).astype(np.float32)
        return r
    raise ValueError(family)


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-identical, NaN anywhere matching NaN (payloads aside)."""
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))


def test_matrix_core_chain_equals_valu_chain_and_oracle():
    rng = np.random.default_rng(11)
    T, H, V = 16, 512, 300          # 2 chunks; V past one 128-row block
    fams = ["normal", "tiny", "huge", "cancel", "zeros"]
    for hf in fams:
        for pf in fams:
            h = _rows(rng, T, H, hf)
            p = _rows(rng, V, H, pf)
            if hf == "cancel" and pf == "cancel":
                p[:, 1::2] = p[:, 0::2]        # products that cancel in pairs
            if hf == "normal" and pf == "huge":
                h[3, 7] = np.inf
                p[5, 100] = np.nan
                h[9, 300] = -np.inf
            ht, pt = _bf16(h).to(DEV), _bf16(p).to(DEV)
            z_mc = M.lm_head_logits(ht, pt).cpu().numpy()          # T > 8: matrix cores
            z_va = np.concatenate([M.lm_head_logits(ht[i:i + 1].contiguous(), pt).cpu().numpy()
                                   for i in range(T)])             # T = 1: VALU
            z_or = O.lm_head_logits(bits(_bf16(h)), bits(_bf16(p)))
            assert _same(z_mc, z_va), (hf, pf, int((z_mc.view(np.uint32) != z_va.view(np.uint32)).sum()))
            assert _same(z_mc, z_or), (hf, pf)
    log(f"[matrix-core chain] {len(fams) ** 2} families of bf16 rows: the K=1 fp32 MFMA chain "
        "== the VALU fma chain == the oracle, bit for bit")


def test_matrix_core_logits_bit_exact_at_layer_shapes():
    """The matrix-core kernel (folded, through the vocabulary-projection entry)
    at the large and tie layers' H and E, on their weight scale, equals the
    oracle bit for bit; the router's own launches at those layers are checked
    through their ids in the route parity tests."""
    from serve_router_gemm_amd import inputs as I
    for name in ("large", "tie"):
        cfg = I.CONFIGS[name]
        T = 96
        x = I.make_tokens(T, cfg.H, 777, "cpu")
        g = torch.Generator().manual_seed(5)
        w = (torch.randn((cfg.E, cfg.H), generator=g) * cfg.w_std).to(torch.bfloat16)
        z = M.lm_head_logits(x.to(DEV), w.to(DEV)).cpu().numpy()
        zr = O.lm_head_logits(bits(x), bits(w))
        assert np.array_equal(z.view(np.uint32), zr.view(np.uint32)), name


def test_matrix_core_logits_ragged_shapes():
    """Partial token and expert blocks and a last chunk narrower than 256
    (H = 2112 ends in a 64-wide chunk), against the oracle bit for bit; the
    one- to four-token shapes and 9-16 tokens over at least 16384 rows run the
    VALU kernels that load whole lines (partial 64-row groups of the
    vocabulary, V below one wave's rows, a last span shorter than 512)."""
    g = torch.Generator().manual_seed(21)
    for T, H, V in ((37, 2112, 200), (70, 320, 129), (9, 64, 1), (1, 2112, 200), (2, 320, 129),
                    (1, 64, 1), (2, 6144, 1000), (4, 2112, 300), (3, 576, 77),
                    (12, 320, 16500), (16, 2112, 16384)):
        h = torch.randn((T, H), generator=g).to(torch.bfloat16)
        p = (torch.randn((V, H), generator=g) * 0.05).to(torch.bfloat16)
        z = M.lm_head_logits(h.to(DEV), p.to(DEV)).cpu().numpy()
        zr = O.lm_head_logits(bits(h), bits(p))
        assert np.array_equal(z.view(np.uint32), zr.view(np.uint32)), (T, H, V)
