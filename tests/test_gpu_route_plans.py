"""The router's launch plans give the same bits (GPU required).

Router logits are fixed-order fp32 chains: 256-wide chunks, each an ascending
fused multiply-add chain from +0, chunk sums added in ascending order
(Fireworks page "位级一致：前沿训练的差异化关键", section
"为什么比特级一致是一个复杂的问题": one reduction order for the router
whatever the batch).  The library picks a launch plan from the batch shape:
the streaming VALU kernel for a few tokens, VALU register tiles (folded, or
one block per chunk), the matrix-core kernel in 4-wave blocks (per chunk or
folded) and, with more than 128 experts and enough tokens to give 256 blocks,
in 8-wave blocks of 64 tokens x 256 experts.  Which plan ran must not show in
any token's experts or weights: each batch is routed whole and in slices that
take the other plans, and every row must agree bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import DEV, gpu, log
from serve_router_gemm_amd import inputs as I

pytestmark = gpu

if torch.cuda.is_available():
    from serve_router_gemm_amd import moe as M

# (name, layer, batch size): the whole batch takes the 8-wave matrix-core plan
CASES = [
    ("large_T16384", I.scaled(I.CONFIGS["large"], F=64), 16384),
    ("E512_k16_T8192", I.scaled(I.CONFIGS["large"], H=512, E=512, k=16, F=64), 8192),
    ("E200_H320_T16384", I.scaled(I.CONFIGS["mid"], H=320, E=200, k=8, F=64), 16384),
]
# slice sizes (other plans) and how many leading tokens each covers
SLICES = [(4096, None), (600, 6000), (128, 2048), (8, 256), (1, 48)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_router_plans_agree_bitwise(case):
    name, cfg, T = case
    L = I.make_layer(cfg, DEV)
    x = I.make_x(cfg, DEV, T)

    def route(xs):
        ids, w = M.route(xs.contiguous(), L["w_router"], cfg.k, cfg.score, cfg.renorm,
                         bias=L["bias"])
        return ids.cpu().numpy(), w.cpu().numpy().view(np.uint32)

    ids0, w0 = route(x)
    for size, cover in SLICES:
        n = min(T, cover or T)
        parts = [route(x[i:min(i + size, n)]) for i in range(0, n, size)]
        ids = np.concatenate([p[0] for p in parts])
        w = np.concatenate([p[1] for p in parts])
        assert np.array_equal(ids, ids0[:n]), (name, size)
        assert np.array_equal(w, w0[:n]), (name, size)
    log(f"[route plans] {name}: ids and weights of the whole batch == slices of "
        f"{', '.join(str(s) for s, _ in SLICES)} tokens, bit for bit")
