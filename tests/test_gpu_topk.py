"""The sparse-indexer top-k on the GPU: index lists equal the oracle's exactly
(heavy ties, NaN, +-inf, +-0, short rows, k up to 4096), and a row's list does
not depend on the other rows of the call."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

from helpers import DEV, gpu, log
from oracle import oracle as O
from serve_router_gemm_amd import moe as M

pytestmark = gpu


def _rows(Q, N, levels, seed):
    rng = np.random.default_rng(seed)
    s = rng.integers(0, levels, size=(Q, N)).astype(np.float32) * np.float32(0.25) - 1.0
    if Q > 0:
        s[0, rng.choice(N, max(1, N // 10), replace=False)] = np.nan
    if Q > 1:
        s[1, : min(N, 5)] = np.inf
        s[1, min(N, 5): min(N, 10)] = -np.inf
    if Q > 2:
        s[2, ::7] = -0.0
        s[2, 1::7] = 0.0
    return s


def _check(s, k, lengths=None):
    st = torch.from_numpy(s).to(DEV)
    lt = None if lengths is None else torch.from_numpy(lengths).to(DEV)
    idx, vals = M.topk_large(st, k, lt)
    ref_idx, ref_vals = O.topk_large(s, k, lengths)
    gi, gv = idx.cpu().numpy(), vals.cpu().numpy()
    assert np.array_equal(gi, ref_idx)
    assert np.array_equal(gv.view(np.uint32), ref_vals.view(np.uint32))
    return gi


@pytest.mark.parametrize("Q,N,k,levels", [
    (6, 1000, 100, 7), (4, 4096, 2048, 50), (3, 131072, 2048, 1000), (5, 300, 300, 3),
    (2, 5000, 4096, 20), (3, 10, 2048, 4), (4, 1, 1, 2), (7, 70000, 1, 100000),
    (3, 20000, 2048, 1)])
def test_topk_large_equals_oracle(Q, N, k, levels):
    _check(_rows(Q, N, levels, N + k), k)


def _randn_rows(Q, N, seed):
    return np.random.default_rng(seed).standard_normal((Q, N)).astype(np.float32)


@pytest.mark.parametrize("Q,N,k", [(4, 131072, 2048), (3, 20000, 4096), (5, 3000, 100),
                                   (2, 70000, 1), (3, 4097, 4096)])
def test_topk_large_continuous_scores(Q, N, k):
    """Continuous scores: the two-read path (the bin of the k-th element and
    those above it hold few elements)."""
    _check(_randn_rows(Q, N, N + k), k)


def test_topk_large_candidates_at_capacity():
    """The two-read path at its capacity: 4096 equal top scores (all of them
    candidates, the top 2048 taken by index) and 4097 (the radix path)."""
    N, k = 50000, 2048
    rng = np.random.default_rng(4)
    s = rng.uniform(-1, 1, (2, N)).astype(np.float32)
    for q, m in ((0, 4096), (1, 4097)):
        s[q, rng.choice(N, m, replace=False)] = 3.0
    gi = _check(s, k)
    assert np.all(np.diff(gi[0]) > 0)              # equal scores: ascending indices


def _sampled_positions(n, q):
    """Positions the kernel samples in row q for its threshold guess: the
    64-score chunks c * stride + rot, c < min(nch, 64),
    stride = nch // min(nch, 64), rot = ((q * 0x9E3779B1 mod 2^32) >> 16)
    mod stride."""
    nch = (n + 63) // 64
    nsc = min(nch, 64)
    stride = nch // nsc
    rot = (((q * 0x9E3779B1) & 0xFFFFFFFF) >> 16) % stride
    ch = np.arange(nsc) * stride + rot
    pos = (ch[:, None] * 64 + np.arange(64)[None, :]).ravel()
    return pos[pos < n]


def test_topk_large_unrepresentative_sample():
    """Rows whose sampled chunks mislead the threshold guess; the list must
    still be the oracle's.  Row 0: the sampled scores are the highest of the
    row, so the guess leaves fewer than k scores.  Row 1: 5000 large,
    spread-out scores sit outside the sample, so the guess leaves more than
    4096 (the exact histogram's two reads follow).  Row 2: the same with 5000
    equal large scores (the radix path follows).  Row 3: a short row whose
    sample is the whole row."""
    Q, N, k = 4, 131072, 2048
    rng = np.random.default_rng(11)
    s = rng.standard_normal((Q, N)).astype(np.float32)
    pos = _sampled_positions(N, 0)
    assert pos.size == 4096
    s[0, pos] = (10.0 + rng.random(pos.size)).astype(np.float32)
    sampled_1_2 = np.union1d(_sampled_positions(N, 1), _sampled_positions(N, 2))
    rest = np.setdiff1d(np.arange(N), sampled_1_2)
    hi = rng.choice(rest, 5000, replace=False)
    s[1, hi] = (2.0 ** rng.uniform(4, 20, hi.size)).astype(np.float32)
    s[2, hi] = 50.0
    lengths = np.array([N, N, N, 3000], dtype=np.int32)
    gi = _check(s, k, lengths)
    assert set(gi[2][:k].tolist()) <= set(hi.tolist())


def test_topk_large_threshold_sign_subnormal_and_infinity():
    """Rows whose k-th score, and so the collection threshold, is negative,
    subnormal, at +-0, or at -inf with NaN below it: the threshold test on
    floats must select what the order code selects."""
    Q, N, k = 5, 40000, 2048
    rng = np.random.default_rng(12)
    s = np.empty((Q, N), dtype=np.float32)
    s[0] = -np.abs(rng.standard_normal(N)).astype(np.float32) - 1.0      # all negative
    s[1] = (rng.standard_normal(N) * 1e-40).astype(np.float32)           # subnormal
    assert np.count_nonzero(np.abs(s[1]) < np.finfo(np.float32).tiny) > N // 2
    s[2] = (-np.abs(rng.standard_normal(N)) * 1e-3).astype(np.float32)  # +-0 at the k-th
    z = rng.choice(N, 7000, replace=False)
    s[2, z[:4000]] = 0.0
    s[2, z[4000:]] = -0.0
    s[2, rng.choice(np.setdiff1d(np.arange(N), z), 1000, replace=False)] = 1.0
    s[3] = -np.inf                                                         # -inf at the k-th
    s[3, rng.choice(N, 1000, replace=False)] = rng.standard_normal(1000).astype(np.float32)
    s[3, rng.choice(N, 5000, replace=False)] = np.nan
    s[4] = np.nan                                                          # NaN at the k-th
    s[4, rng.choice(N, 100, replace=False)] = -np.inf
    _check(s, k)


def test_topk_large_continuous_causal():
    Q, N, k = 8, 9000, 2048
    s = _randn_rows(Q, N, 77)
    lengths = np.array([0, 5, 2048, 2049, 4000, 8999, 9000, 6000], dtype=np.int32)
    _check(s, k, lengths)


def test_topk_large_causal_lengths():
    Q, N, k = 16, 9000, 2048
    s = _rows(Q, N, 300, 5)
    lengths = np.array([0, 1, 2, 100, 2047, 2048, 2049, 4000, 8999, 9000, 9001, -3, 5000,
                        3000, 2500, 7000], dtype=np.int32)
    gi = _check(s, k, lengths)
    assert np.all(gi[0] == -1)


def test_topk_large_row_does_not_depend_on_batch():
    Q, N, k = 32, 65536, 2048
    s = _rows(Q, N, 5000, 9)
    st = torch.from_numpy(s).to(DEV)
    full, _ = M.topk_large(st, k)
    for q in (0, 7, 31):
        one, _ = M.topk_large(st[q:q + 1].contiguous(), k)
        assert torch.equal(one[0], full[q]), q
    # a shuffled batch gives the same rows
    perm = torch.randperm(Q, generator=torch.Generator().manual_seed(1)).to(DEV)
    sh, _ = M.topk_large(st[perm].contiguous(), k)
    assert torch.equal(sh, full[perm])


def test_topk_large_timing_indexer_shape():
    """Indexer shape: 1024 queries x 131072 keys, top 2048 (logged, not asserted)."""
    Q, N, k = 1024, 131072, 2048
    st = torch.randn((Q, N), generator=torch.Generator().manual_seed(3)).to(DEV)
    M.topk_large(st, k, want_vals=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        M.topk_large(st, k, want_vals=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000 / 3
    log(f"[topk] Q={Q} N={N} k={k}: {ms:.3f} ms, {Q * N * 4 / ms / 1e6:.1f} GB/s of scores")
