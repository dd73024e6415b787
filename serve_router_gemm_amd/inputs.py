"""Seeded synthetic inputs for the MoE layer forward.

This module only draws and lays out input bytes (weights, hidden states,
router bias, constructed tie cases).  It holds none of the layer's arithmetic,
so both the HIP path and the CPU oracle can consume the same bytes.

Layouts (bf16 tensors hold bfloat16 values, row-major, K contiguous):
  x        [T, H]     bf16   hidden states
  w_router [E, H]     bf16
  w_gate   [E, F, H]  bf16
  w_up     [E, F, H]  bf16
  w_down   [E, H, F]  bf16
  bias     [E]        fp32   (sigmoid scoring only; selection only)

Workload shapes follow the MoE layers the pages discuss (Fireworks, "Bit-level
agreement" page, section on why bit-level agreement is hard: router near-ties
and per-expert token counts that depend on the co-batch).  The pages give no
sizes; the five layer presets below are the synthetic stand-ins.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int
    E: int
    k: int
    F: int
    score: int
    renorm: bool
    w_std: float
    T: int
    seed: int = 0
    zipf_s: float = 0.0     # >0: sigmoid bias skews expert load like Zipf(s)
    kappa: float = 0.1      # bias scale for the Zipf skew

    @property
    def A(self) -> int:
        return self.T * self.k


CONFIGS = {
    # small case: every token, every stage through the oracle in well under a second
    "tiny": LayerConfig("tiny", H=256, E=8, k=2, F=512, score=SCORE_SOFTMAX,
                        renorm=True, w_std=0.02, T=64),
    # batch-invariance sweep layer; T is swept over {1, 7, 128, 1024, 4096}
    "mid": LayerConfig("mid", H=2048, E=64, k=8, F=1408, score=SCORE_SOFTMAX,
                       renorm=True, w_std=0.02, T=4096),
    # large layer: sigmoid scores, Zipf(1.2)-skewed expert load via the bias
    "large": LayerConfig("large", H=6144, E=256, k=8, F=2048, score=SCORE_SIGMOID,
                         renorm=True, w_std=0.01, T=16384, zipf_s=1.2, kappa=0.1),
    # near-tie routing stress: constructed exact ties and 1-ulp gaps
    "tie": LayerConfig("tie", H=4096, E=128, k=8, F=2048, score=SCORE_SOFTMAX,
                       renorm=True, w_std=0.02, T=8192),
    # decode-shaped steps on the large layer; T is swept over {1, 4, 16, 64}
    "dec": LayerConfig("dec", H=6144, E=256, k=8, F=2048, score=SCORE_SIGMOID,
                       renorm=True, w_std=0.01, T=64, zipf_s=1.2, kappa=0.1),
}

MID_SWEEP_T = (1, 7, 128, 1024, 4096)
DEC_SWEEP_T = (1, 4, 16, 64)
TIE_SWEEP_T = (1, 64, 1024, 8192)

PROBE_SEED = 7
COTOKEN_SEED_BASE = 1000
PROJ_SEED = 11


def scaled(cfg: LayerConfig, **kw) -> LayerConfig:
    """The same layer family with some sizes replaced (used for small test cases)."""
    return dataclasses.replace(cfg, **kw)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, std, gen, device, chunk_rows=None) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and rounded to bf16 (round-to-nearest-even).

    Drawn in chunks along dim 0 so a 19 GB weight tensor never needs an fp32 copy.
    """
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n0 = shape[0]
    step = chunk_rows or n0
    for s in range(0, n0, step):
        e = min(n0, s + step)
        t = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        out[s:e].copy_(t)
        del t
    return out


def zipf_bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert selection bias b_e = -kappa * s * ln(rank_e), ranks a seeded permutation.

    With sigmoid scores this skews expert load so that a few experts take
    thousands of tokens and many take none.
    """
    rng = np.random.default_rng(cfg.seed + 2)
    ranks = rng.permutation(cfg.E) + 1
    return (-cfg.kappa * cfg.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)


def make_layer(cfg: LayerConfig, device="cpu") -> dict:
    """Layer weights for `cfg`, drawn in the order w_router, w_gate, w_up, w_down."""
    device = torch.device(device)
    g = _gen(device, cfg.seed)
    E, H, F = cfg.E, cfg.H, cfg.F
    # one expert per chunk bounds the fp32 staging buffer to a single expert
    wr = _randn_bf16((E, H), cfg.w_std, g, device)
    wg = _randn_bf16((E, F, H), cfg.w_std, g, device, chunk_rows=1)
    wu = _randn_bf16((E, F, H), cfg.w_std, g, device, chunk_rows=1)
    wd = _randn_bf16((E, H, F), cfg.w_std, g, device, chunk_rows=1)
    bias = None
    if cfg.score == SCORE_SIGMOID:
        bias = torch.from_numpy(zipf_bias(cfg)).to(device) if cfg.zipf_s > 0 else \
            torch.zeros(E, dtype=torch.float32, device=device)
    return dict(w_router=wr, w_gate=wg, w_up=wu, w_down=wd, bias=bias)


def make_tokens(n: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    """n hidden-state rows, N(0,1) rounded to bf16."""
    device = torch.device(device)
    if n == 0:
        return torch.empty((0, H), dtype=torch.bfloat16, device=device)
    return _randn_bf16((n, H), 1.0, _gen(device, seed), device)


def make_x(cfg: LayerConfig, device="cpu", T: int | None = None) -> torch.Tensor:
    return make_tokens(cfg.T if T is None else T, cfg.H, cfg.seed + 1, device)


def probes(H: int, n: int = 16, device="cpu") -> torch.Tensor:
    """The fixed probe tokens: the same bytes whatever batch they are placed in."""
    return make_tokens(n, H, PROBE_SEED, "cpu").to(device)


def embed_probes(probe_rows: torch.Tensor, T: int, rep: int, seed_offset: int = 0):
    """A batch of T rows that contains every probe row at seeded positions.

    The other rows are fresh N(0,1) co-tokens from seed COTOKEN_SEED_BASE + rep.
    Returns (x [T, H], positions [n_probes]).
    """
    n, H = probe_rows.shape
    assert T >= n
    dev = probe_rows.device
    x = make_tokens(T, H, COTOKEN_SEED_BASE + rep + seed_offset, "cpu").to(dev)
    rng = np.random.default_rng(COTOKEN_SEED_BASE + 31 * rep + seed_offset)
    pos = np.sort(rng.choice(T, size=n, replace=False)) if rep % 2 == 0 else \
        rng.choice(T, size=n, replace=False)
    pos_t = torch.from_numpy(pos.astype(np.int64)).to(dev)
    x[pos_t] = probe_rows
    return x, pos


# ----------------------------------------------------------------------------
# near-tie routing stress inputs
# ----------------------------------------------------------------------------

def _trunc_bf16_f32(v: np.ndarray) -> np.ndarray:
    """Truncate fp32 values to their top 16 bits (a bf16 value, toward zero)."""
    b = v.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32)


def split_to_bf16_triple(z: np.ndarray):
    """Write each fp32 z as a + b*2^-8 + c*2^-16 with a, b, c exact bf16 values.

    a keeps z's top 8 significant bits, b the next 8, c the last 8, so every
    partial sum of the three terms is exactly representable in fp32.
    """
    z = z.astype(np.float32)
    a = _trunc_bf16_f32(z)
    r1 = (z - a).astype(np.float32)              # exact: <= 16 significant bits
    r1s = (r1 * np.float32(256.0)).astype(np.float32)
    b = _trunc_bf16_f32(r1s)
    c = ((r1s - b) * np.float32(256.0)).astype(np.float32)
    assert np.array_equal(_trunc_bf16_f32(c), c), "c must be an exact bf16 value"
    return a, b, c


def make_tie_inputs(cfg: LayerConfig, T: int | None = None, seed: int | None = None):
    """Router weights and tokens with exactly-known logits for the near-tie stress.

    Router rows: w[e, e] = 1, w[e, E+e] = 2^-8, w[e, 2E+e] = 2^-16, other entries
    of the first 3E columns 0, columns >= 3E drawn N(0, w_std^2).
    Token kinds (by index mod 4): 0,1 random N(0,1) rows; 2 exact tie at the
    k-th / (k+1)-th boundary; 3 the (k+1)-th one fp32 ulp below the k-th.
    A stress token has x[3E:] = 0 and x[e], x[E+e], x[2E+e] = the bf16 triple
    of its target logit z_e, so its logit for expert e equals z_e exactly under
    any summation order.

    Returns dict(w_router [E,H] bf16, x [T,H] bf16, kind [T] int, z [T,E] fp32)
    with z only meaningful for stress tokens.
    """
    E, H, k = cfg.E, cfg.H, cfg.k
    T = cfg.T if T is None else T
    assert 3 * E <= H
    rng = np.random.default_rng(cfg.seed + 5 if seed is None else seed)
    wr = np.zeros((E, H), dtype=np.float32)
    wr[:, 3 * E:] = rng.standard_normal((E, H - 3 * E), dtype=np.float32) * np.float32(cfg.w_std)
    for e in range(E):
        wr[e, e] = 1.0
        wr[e, E + e] = 2.0 ** -8
        wr[e, 2 * E + e] = 2.0 ** -16
    wr_bf = torch.from_numpy(wr).to(torch.bfloat16)

    kind = np.arange(T) % 4
    x = torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16)
    z = rng.standard_normal((T, E), dtype=np.float32)
    stress = np.nonzero(kind >= 2)[0]
    for t in stress:
        zt = z[t]
        order = np.argsort(-zt, kind="stable")
        ek = order[k - 1]
        ek1 = order[k] if k < E else None
        if ek1 is not None:
            if kind[t] == 2:
                zt[ek1] = zt[ek]
            else:
                zt[ek1] = np.nextafter(zt[ek], np.float32(-np.inf), dtype=np.float32)
        a, b, c = split_to_bf16_triple(zt)
        row = np.zeros(H, dtype=np.float32)
        row[0:E] = a
        row[E:2 * E] = b
        row[2 * E:3 * E] = c
        xr = torch.from_numpy(row).to(torch.bfloat16)
        assert torch.equal(xr.float(), torch.from_numpy(row)), "triple must be exact bf16"
        x[t] = xr
    return dict(w_router=wr_bf, x=x, kind=kind, z=z)


# ----------------------------------------------------------------------------
# host views for the oracle
# ----------------------------------------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 numpy view of a bf16 tensor's bit patterns (copied to host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def describe(cfg: LayerConfig) -> str:
    return (f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} F={cfg.F} "
            f"score={'softmax' if cfg.score == SCORE_SOFTMAX else 'sigmoid'} "
            f"renorm={int(cfg.renorm)} w_std={cfg.w_std}")


def expert_flops(cfg: LayerConfig, T: int | None = None) -> float:
    """Algorithmic flops of the expert FFN: 6*H*F per assignment (no padding)."""
    T = cfg.T if T is None else T
    return 6.0 * T * cfg.k * cfg.H * cfg.F

