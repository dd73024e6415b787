"""Router replay on the GPU: replaying moe_forward's own routing reproduces its
output bit for bit (recorded or recomputed weights), other expert choices match
the oracle's replay, and ids outside [0,E) contribute nothing."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import DEV, assert_out_close, bits, gpu, host, layer, log, weights_close
from oracle import oracle as O
from serve_router_gemm_amd import inputs as I
from serve_router_gemm_amd import moe as M

pytestmark = gpu


def _cfg(name, **kw):
    return I.scaled(I.CONFIGS[name], **kw)


def _routed(cfg, L, x, variant=0):
    return M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score,
                     cfg.renorm, bias=L["bias"], variant=variant, return_routing=True)


@pytest.mark.parametrize("name,T", [("tiny", 64), ("mid", 300), ("large", 512), ("tie", 257)])
def test_replay_of_own_routing_is_bit_identical(name, T):
    cfg = _cfg(name, T=T)
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    out, ids, w = _routed(cfg, L, x)
    rec = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"], topk_w=w,
                           score=cfg.score, renormalize=cfg.renorm)
    assert torch.equal(rec.view(torch.int16), out.view(torch.int16))
    rep, w2 = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"],
                               w_router=L["w_router"], score=cfg.score,
                               renormalize=cfg.renorm, return_weights=True)
    assert torch.equal(w2.view(torch.int32), w.view(torch.int32))
    assert torch.equal(rep.view(torch.int16), out.view(torch.int16))
    # The load-dependent variant is deterministic for a given routing (its
    # splits follow the per-expert counts, and its parts are added in a fixed
    # order): its replay reproduces its routed run bit for bit too.
    out_v, ids_v, w_v = _routed(cfg, L, x, variant=1)
    rep_v = M.forward_replay(x, ids_v, L["w_gate"], L["w_up"], L["w_down"], topk_w=w_v,
                             score=cfg.score, renormalize=cfg.renorm, variant=1)
    assert torch.equal(rep_v.view(torch.int16), out_v.view(torch.int16))


@pytest.mark.parametrize("name,T", [("tiny", 64), ("mid", 200)])
def test_replay_of_other_experts_matches_oracle(name, T):
    cfg = _cfg(name, T=T)
    L = layer(cfg)
    hb = host(cfg)
    x = I.make_x(cfg, DEV)
    rng = np.random.default_rng(5)
    ids_np = rng.integers(0, cfg.E, size=(T, cfg.k)).astype(np.int32)
    ids_np[::5, -1] = -1                       # some slots recorded as "none"
    ids_np[3::7, 0] = cfg.E + 2
    ids = torch.from_numpy(ids_np).to(DEV)
    out, w = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"],
                              w_router=L["w_router"], score=cfg.score, renormalize=cfg.renorm,
                              return_weights=True)
    ref_out, ref_w = O.forward_replay(bits(x), hb["w_router"], ids_np, hb["w_gate"],
                                      hb["w_up"], hb["w_down"], cfg.score, cfg.renorm)
    weights_close(w.cpu().numpy(), ref_w)
    assert np.all(w.cpu().numpy()[(ids_np < 0) | (ids_np >= cfg.E)] == 0.0)
    stats = assert_out_close(bits(out), ref_out, what=f"replay {name}")
    log(f"[replay] {name} T={T}: {stats}")
    # recorded weights are used as given
    w_rec = torch.rand((T, cfg.k), generator=torch.Generator().manual_seed(1)).to(DEV)
    out2 = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"], topk_w=w_rec,
                            score=cfg.score, renormalize=cfg.renorm)
    ref2, _ = O.forward_replay(bits(x), None, ids_np, hb["w_gate"], hb["w_up"], hb["w_down"],
                               cfg.score, cfg.renorm, w=w_rec.cpu().numpy())
    assert_out_close(bits(out2), ref2, what=f"replay recorded w {name}")


def test_replay_is_batch_invariant():
    cfg = _cfg("mid", T=1024)
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    rng = np.random.default_rng(9)
    ids = torch.from_numpy(rng.integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)).to(DEV)
    full = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"], w_router=L["w_router"],
                            score=cfg.score, renormalize=cfg.renorm)
    for t in (0, 517, 1023):
        one = M.forward_replay(x[t:t + 1].contiguous(), ids[t:t + 1].contiguous(), L["w_gate"],
                               L["w_up"], L["w_down"], w_router=L["w_router"], score=cfg.score,
                               renormalize=cfg.renorm)
        assert torch.equal(one.view(torch.int16), full[t:t + 1].view(torch.int16)), t


def test_replay_with_repeated_experts_small_batch():
    """Recorded ids that repeat an expert inside a token (the router never
    does): in a 12-token batch expert 3 gets 20 rows, more than one 16-row
    chunk of the weight-streaming GEMM, and the result matches the oracle's
    replay (each slot evaluated on its own)."""
    cfg = _cfg("tiny", T=12)
    L = layer(cfg)
    hb = host(cfg)
    x = I.make_x(cfg, DEV)
    rng = np.random.default_rng(21)
    ids_np = rng.integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)
    ids_np[:10, :] = 3
    ids = torch.from_numpy(ids_np).to(DEV)
    out, w = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"],
                              w_router=L["w_router"], score=cfg.score, renormalize=cfg.renorm,
                              return_weights=True)
    ref_out, ref_w = O.forward_replay(bits(x), hb["w_router"], ids_np, hb["w_gate"],
                                      hb["w_up"], hb["w_down"], cfg.score, cfg.renorm)
    weights_close(w.cpu().numpy(), ref_w)
    stats = assert_out_close(bits(out), ref_out, what="replay repeated experts")
    log(f"[replay] repeated experts, T=12: {stats}")
