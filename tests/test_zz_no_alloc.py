"""moe_forward_static (the layer with the library's static per-GPU scratch
instead of a caller workspace) against moe_forward, through the C ABI: out,
topk_ids and topk_w bit-identical on two calls in a row, the second with a
smaller batch, for the decode layer and the mid layer; sizes beyond the
scratch are rejected; the call leaves torch's allocator untouched."""
from __future__ import annotations

import pytest
import torch

from helpers import DEV, gpu, layer, log
from serve_router_gemm_amd import inputs as I

pytestmark = gpu

if torch.cuda.is_available():
    from serve_router_gemm_amd import moe as M


def _static_vs_forward(cfg, T, seed, variant=0):
    L = layer(cfg)
    x = I.make_tokens(T, cfg.H, seed, "cpu").to(DEV)
    ref, ids_r, w_r = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k,
                                cfg.score, cfg.renorm, bias=L["bias"], variant=variant,
                                return_routing=True)
    out = torch.empty_like(ref)
    ids = torch.empty_like(ids_r)
    w = torch.empty_like(w_r)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    M.forward_static(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score,
                     cfg.renorm, bias=L["bias"], variant=variant, out=out, topk_ids=ids,
                     topk_w=w)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(ids, ids_r), (cfg.name, T)
    assert torch.equal(w.view(torch.int32), w_r.view(torch.int32)), (cfg.name, T)
    if variant == 0:
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (cfg.name, T)
    return out


@pytest.mark.parametrize("name,T1,T2", [("dec", 132, 7), ("mid", 371, 64), ("tiny", 64, 1)])
def test_forward_static_matches_forward(name, T1, T2):
    cfg = I.CONFIGS[name]
    log(f"[static] {name}: T = {T1} then T = {T2}")
    _static_vs_forward(cfg, T1, 4242 + T1)
    _static_vs_forward(cfg, T2, 4343 + T2)


def test_forward_static_variant_routing_and_rejection():
    cfg = I.CONFIGS["dec"]
    log("[static] dec: split-K variant routing, then a batch beyond the scratch")
    _static_vs_forward(cfg, 16, 77, variant=1)
    L = layer(cfg)
    x = I.make_tokens(133, cfg.H, 5, "cpu").to(DEV)
    with pytest.raises(M.MoeError) as e:
        M.forward_static(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], cfg.k, cfg.score,
                         cfg.renorm, bias=L["bias"])
    assert e.value.rc == -7
