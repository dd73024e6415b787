"""The layer forward captured as one HIP graph and replayed.

A decode step is a handful of short launches, so launch gaps weigh on it;
serving loops replay such a step as a captured graph.  Nothing in the path
allocates, copies or sets memory (`moe_forward` takes its workspace,
`moe_forward_static` its static scratch), so the capture holds the kernels
only.  Every replay must give the eager result bit for bit, with eager work
and synchronisations between replays (the same layer, the same bits whatever
launches it: Fireworks page "位级一致：前沿训练的差异化关键", section
"曾经只有前沿实验室才有的功能")."""
from __future__ import annotations

import pytest
import torch

from helpers import DEV, gpu, layer, log
from serve_router_gemm_amd import inputs as I
from serve_router_gemm_amd import moe as M

pytestmark = gpu

CASES = [("dec", 1), ("dec", 64), ("mid", 7), ("mid", 1024)]


def _capture(fn) -> torch.cuda.CUDAGraph:
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                # warm up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("name,T", CASES, ids=lambda v: str(v))
def test_forward_graph_replays_bit_identical(name, T):
    cfg = I.scaled(I.CONFIGS[name], T=T)
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    args = (x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score, cfg.renorm)
    eager = M.forward(*args, bias=L["bias"])
    out = torch.empty_like(eager)
    ws = M.workspace(M.OP_FORWARD, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k)
    g = _capture(lambda: M.forward(*args, bias=L["bias"], out=out, ws=ws))
    for r in range(4):
        out.fill_(0.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (name, T, r)
    del g
    log(f"[graph] {name} T={T}: 4 replays of the captured forward == eager, bit for bit")


@pytest.mark.parametrize("name,T", [("dec", 1), ("dec", 64)], ids=lambda v: str(v))
def test_forward_static_graph_replays_bit_identical(name, T):
    cfg = I.scaled(I.CONFIGS[name], T=T)
    L = layer(cfg)
    x = I.make_x(cfg, DEV)
    args = (x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score, cfg.renorm)
    eager = M.forward(*args, bias=L["bias"])
    out = torch.empty_like(eager)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    g = _capture(lambda: M.forward_static(*args, bias=L["bias"], out=out, topk_ids=ids, topk_w=w))
    for r in range(4):
        out.fill_(0.0)
        # an eager call of the same entry between replays (it shares the scratch)
        M.forward_static(*args, bias=L["bias"], out=torch.empty_like(out))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), (name, T, r)
    del g
