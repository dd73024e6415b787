"""ctypes wrapper of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg.  It never imports the HIP library or its
binding, and the product path never imports it.

All arrays are numpy; bf16 tensors travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

SOFTMAX = 0
SIGMOID = 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            # the checker is plain C; build it on first use if nobody has
            from oracle import build as _b
            _b.build(verbose=False)
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


def _declare(L):
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    i64 = ctypes.c_int64
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_f32_to_bf16.restype = ctypes.c_uint16
    L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    L.orc_f32_to_bf16_array.argtypes = [P, P, i64]
    L.orc_max_threads.restype = i32
    L.orc_router_logits.argtypes = [i32, i32, i32, P, P, P, i32]
    L.orc_topk_keys.argtypes = [i32, i32, i32, P, P]
    L.orc_route.restype = i32
    L.orc_route.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, i32]
    L.orc_permute.restype = i32
    L.orc_permute.argtypes = [i32, i32, P, P, P, P, P]
    L.orc_expert_ffn.restype = i32
    L.orc_expert_ffn.argtypes = [i32, P, P, i32, i32, i32, P, P, P, P, P, P, i32]
    L.orc_expert_down.restype = i32
    L.orc_expert_down.argtypes = [i32, P, i32, i32, i32, P, P, P, i32]
    L.orc_combine.argtypes = [i32, i32, i32, P, P, P]
    L.orc_forward.restype = i32
    L.orc_forward.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                              P, P, P, P, P, P, P, P, i32]
    L.orc_forward_tokens.restype = i32
    L.orc_forward_tokens.argtypes = [i32, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                     P, P, P, P, P, i32]
    L.orc_replay_weights.restype = i32
    L.orc_replay_weights.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, i32]
    L.orc_forward_replay.restype = i32
    L.orc_forward_replay.argtypes = [i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P,
                                     P, i32]
    L.orc_lm_head_logits.argtypes = [i32, i32, i32, P, P, P, i32]
    L.orc_topk_large.argtypes = [i32, i32, i32, P, P, P, P, i32]
    L.orc_e4m3_to_f32.restype = ctypes.c_float
    L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.orc_f32_to_e4m3_array.argtypes = [P, P, i64]
    L.orc_fp8_block_exp.restype = i32
    L.orc_fp8_block_exp.argtypes = [ctypes.c_float]
    L.orc_quantize_fp8.argtypes = [i32, i32, i32, P, P, P]
    L.orc_expert_ffn_fp8.restype = i32
    L.orc_expert_ffn_fp8.argtypes = [i32, P, P, i32, i32, P, P, P, P, P, P, P, P, P, P, i32]
    L.orc_fp8_gemm.restype = i32
    L.orc_fp8_gemm.argtypes = [i32, i32, i32, P, P, P, P, P, P, i32]
    L.orc_forward_tokens_fp8.restype = i32
    L.orc_forward_tokens_fp8.argtypes = [i32, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P,
                                         P, P, P, P, P, P, P, P, P, i32]
    L.orc_log_softmax.argtypes = [i32, i32, P, P, i32]
    L.orc_exp32.restype = ctypes.c_float
    L.orc_exp32.argtypes = [ctypes.c_float]
    L.orc_log32.restype = ctypes.c_float
    L.orc_log32.argtypes = [ctypes.c_float]
    L.orc_k3.argtypes = [i32, i32, P, P, P, P, P]


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def max_threads() -> int:
    return int(lib().orc_max_threads())


def f32_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_p(v), _p(out), v.size)
    return out


def bf16_to_f32(b) -> np.ndarray:
    b = _u16(b)
    return (b.astype(np.uint32) << 16).view(np.float32)


def router_logits(x, wr, nthreads=0) -> np.ndarray:
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(T, H, E, _p(x), _p(wr), _p(out), nthreads)
    return out


def topk_keys(keys, k) -> np.ndarray:
    keys = _c(keys, np.float32)
    n, E = keys.shape
    ids = np.empty((n, k), dtype=np.int32)
    lib().orc_topk_keys(n, E, k, _p(keys), _p(ids))
    return ids


def route(x, wr, k, score, renorm=True, bias=None, nthreads=0):
    """-> (ids [T,k] int32, w [T,k] fp32, gap [T] fp64)"""
    x, wr = _u16(x), _u16(wr)
    T, H = x.shape
    E = wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    gap = np.empty((T,), dtype=np.float64)
    rc = lib().orc_route(T, H, E, k, score, int(renorm), _p(x), _p(wr), _p(b), _p(ids), _p(w),
                         _p(gap), nthreads)
    if rc != 0:
        raise ValueError(f"orc_route rc={rc}")
    return ids, w, gap


def permute(ids, E):
    """-> (counts [E], offsets [E+1], perm [A], inv_perm [A]) all int32"""
    ids = _c(ids, np.int32).reshape(-1)
    A = ids.size
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(A, dtype=np.int32)
    inv = np.empty(A, dtype=np.int32)
    rc = lib().orc_permute(A, E, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv))
    if rc != 0:
        raise ValueError(f"orc_permute rc={rc}")
    return counts, offsets, perm, inv


def expert_ffn(tokens, experts, x, wg, wu, wd, want_act=False, nthreads=0):
    """(token, expert) pairs -> y [n,H] fp32 (and act [n,F] bf16 bits)."""
    x, wg, wu, wd = _u16(x), _u16(wg), _u16(wu), _u16(wd)
    tokens = _c(tokens, np.int32).reshape(-1)
    experts = _c(experts, np.int32).reshape(-1)
    n = tokens.size
    H = x.shape[1]
    E, F = wg.shape[0], wg.shape[1]
    y = np.empty((n, H), dtype=np.float32)
    act = np.empty((n, F), dtype=np.uint16) if want_act else None
    rc = lib().orc_expert_ffn(n, _p(tokens), _p(experts), H, E, F, _p(x), _p(wg), _p(wu),
                              _p(wd), _p(act), _p(y), nthreads)
    if rc != 0:
        raise ValueError(f"orc_expert_ffn rc={rc}")
    return (y, act) if want_act else y


def expert_down(experts, act, wd, nthreads=0) -> np.ndarray:
    """Down projection of given act rows (bf16 bits [n,F]) -> y [n,H] fp32."""
    act, wd = _u16(act), _u16(wd)
    experts = _c(experts, np.int32).reshape(-1)
    n, F = act.shape
    E, H = wd.shape[0], wd.shape[1]
    assert wd.shape[2] == F and experts.size == n
    y = np.empty((n, H), dtype=np.float32)
    rc = lib().orc_expert_down(n, _p(experts), H, E, F, _p(act), _p(wd), _p(y), nthreads)
    if rc != 0:
        raise ValueError(f"orc_expert_down rc={rc}")
    return y


def combine(y, w, T, H, k) -> np.ndarray:
    y = _c(y, np.float32)
    w = _c(w, np.float32)
    assert y.size == T * k * H and w.size == T * k
    out = np.empty((T, H), dtype=np.uint16)
    lib().orc_combine(T, H, k, _p(y), _p(w), _p(out))
    return out


def forward(x, wr, wg, wu, wd, k, score, renorm=True, bias=None, nthreads=0, want_y=True):
    """The whole layer in the method's order.  Returns a dict of numpy arrays."""
    x, wr, wg, wu, wd = _u16(x), _u16(wr), _u16(wg), _u16(wu), _u16(wd)
    T, H = x.shape
    E, F = wg.shape[0], wg.shape[1]
    A = T * k
    b = None if bias is None else _c(bias, np.float32)
    r = dict(out=np.empty((T, H), dtype=np.uint16), ids=np.empty((T, k), dtype=np.int32),
             w=np.empty((T, k), dtype=np.float32), gap=np.empty(T, dtype=np.float64),
             counts=np.empty(E, dtype=np.int32), offsets=np.empty(E + 1, dtype=np.int32),
             perm=np.empty(A, dtype=np.int32), inv_perm=np.empty(A, dtype=np.int32),
             y=np.empty((A, H), dtype=np.float32) if want_y else None)
    rc = lib().orc_forward(T, H, E, F, k, score, int(renorm), _p(x), _p(wr), _p(b), _p(wg),
                           _p(wu), _p(wd), _p(r["out"]), _p(r["ids"]), _p(r["w"]),
                           _p(r["gap"]), _p(r["counts"]), _p(r["offsets"]), _p(r["perm"]),
                           _p(r["inv_perm"]), _p(r["y"]), nthreads)
    if rc != 0:
        raise ValueError(f"orc_forward rc={rc}")
    return r


def forward_tokens(tokens, x, wr, wg, wu, wd, k, score, renorm=True, bias=None, nthreads=0):
    """Per-token evaluation of the chosen rows.  -> (out [n,H] bf16 bits, ids, w, gap)"""
    x, wr, wg, wu, wd = _u16(x), _u16(wr), _u16(wg), _u16(wu), _u16(wd)
    tokens = _c(tokens, np.int32).reshape(-1)
    n = tokens.size
    H = x.shape[1]
    E, F = wg.shape[0], wg.shape[1]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((n, H), dtype=np.uint16)
    ids = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float32)
    gap = np.empty(n, dtype=np.float64)
    rc = lib().orc_forward_tokens(n, _p(tokens), H, E, F, k, score, int(renorm), _p(x), _p(wr),
                                  _p(b), _p(wg), _p(wu), _p(wd), _p(out), _p(ids), _p(w),
                                  _p(gap), nthreads)
    if rc != 0:
        raise ValueError(f"orc_forward_tokens rc={rc}")
    return out, ids, w, gap


# ---------------------------------------------------------------------------
# D8: downstream measurement of a decode step (LM head, log-softmax, k3)
# ---------------------------------------------------------------------------

def lm_head_logits(h, proj, nthreads=0) -> np.ndarray:
    """z [T,V] fp32 of bf16 rows h [T,H] against a bf16 projection [V,H], in the
    pinned chunked order of the router logits."""
    h, proj = _u16(h), _u16(proj)
    T, H = h.shape
    V = proj.shape[0]
    z = np.empty((T, V), dtype=np.float32)
    lib().orc_lm_head_logits(T, H, V, _p(h), _p(proj), _p(z), nthreads)
    return z


def log_softmax(z, nthreads=0) -> np.ndarray:
    """fp32 log-softmax over the last axis with fixed chunked sums."""
    z = _c(z, np.float32)
    T, V = z.shape
    out = np.empty_like(z)
    lib().orc_log_softmax(T, V, _p(z), _p(out), nthreads)
    return out


def exp32(a: float) -> np.float32:
    """The correctly rounded fp32 exponential of the log-softmax definition."""
    return np.float32(lib().orc_exp32(float(np.float32(a))))


def log32(a: float) -> np.float32:
    """The correctly rounded fp32 logarithm of the log-softmax definition."""
    return np.float32(lib().orc_log32(float(np.float32(a))))


def k3(logp_ref, logp_test):
    """Schulman's k3 per row: (mean over p_test in fp64, k3 at the greedy token,
    greedy token index)."""
    r = _c(logp_ref, np.float32)
    q = _c(logp_test, np.float32)
    assert r.shape == q.shape and r.ndim == 2
    T, V = q.shape
    mean = np.empty(T, dtype=np.float64)
    gk3 = np.empty(T, dtype=np.float64)
    g = np.empty(T, dtype=np.int32)
    lib().orc_k3(T, V, _p(r), _p(q), _p(mean), _p(gk3), _p(g))
    return mean, gk3, g


# ---------------------------------------------------------------------------
# router replay
# ---------------------------------------------------------------------------

def replay_weights(x, wr, ids, score, renorm=True, nthreads=0) -> np.ndarray:
    """D4 weights of the given experts ids [T,k] (ids outside [0,E) get 0)."""
    x, wr = _u16(x), _u16(wr)
    ids = _c(ids, np.int32)
    T, H = x.shape
    E = wr.shape[0]
    k = ids.shape[1]
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().orc_replay_weights(T, H, E, k, score, int(renorm), _p(x), _p(wr), _p(ids), _p(w),
                                  nthreads)
    if rc != 0:
        raise ValueError(f"orc_replay_weights rc={rc}")
    return w


def forward_replay(x, wr, ids, wg, wu, wd, score, renorm=True, w=None, nthreads=0):
    """The layer with the experts given (router replay): -> (out bf16 bits, weights used)."""
    x, wg, wu, wd = _u16(x), _u16(wg), _u16(wu), _u16(wd)
    wr = None if wr is None else _u16(wr)
    ids = _c(ids, np.int32)
    T, H = x.shape
    E, F = wg.shape[0], wg.shape[1]
    k = ids.shape[1]
    w_in = None if w is None else _c(w, np.float32)
    out = np.empty((T, H), dtype=np.uint16)
    w_out = np.empty((T, k), dtype=np.float32)
    rc = lib().orc_forward_replay(T, H, E, F, k, score, int(renorm), _p(x), _p(wr), _p(ids),
                                  _p(w_in), _p(wg), _p(wu), _p(wd), _p(out), _p(w_out), nthreads)
    if rc != 0:
        raise ValueError(f"orc_forward_replay rc={rc}")
    return out, w_out


# ---------------------------------------------------------------------------
# large-k top-k (sparse attention indexer selection)
# ---------------------------------------------------------------------------

def topk_large(scores, k, lengths=None, nthreads=0):
    """Top k of each row of scores [Q,N] (fp32) under the selection order of
    D3, over the first lengths[q] entries: -> (idx [Q,k] int32, vals [Q,k])."""
    s = _c(scores, np.float32)
    Q, N = s.shape
    ln = None if lengths is None else _c(lengths, np.int32)
    idx = np.empty((Q, k), dtype=np.int32)
    vals = np.empty((Q, k), dtype=np.float32)
    lib().orc_topk_large(Q, N, k, _p(s), _p(ln), _p(idx), _p(vals), nthreads)
    return idx, vals


# ---------------------------------------------------------------------------
# FP8 rollout path (e4m3 experts, power-of-two block scales)
# ---------------------------------------------------------------------------
FP8_BLOCK = 128


def e4m3_to_f32(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    table = np.array([lib().orc_e4m3_to_f32(i) for i in range(256)], dtype=np.float32)
    return table[c]


def f32_to_e4m3(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_f32_to_e4m3_array(_p(v), _p(out), v.size)
    return out


def fp8_block_exp(amax: float) -> int:
    return int(lib().orc_fp8_block_exp(float(amax)))


def quantize_fp8(src, block_rows):
    """bf16 bits [..., R, K] -> (codes uint8 [..., R, K], exps int8 [..., R/block_rows, K/128]),
    each leading index quantised on its own."""
    s = _u16(src)
    *lead, R, K = s.shape
    s2 = s.reshape(-1, R, K)
    q = np.empty(s2.shape, dtype=np.uint8)
    e = np.empty((s2.shape[0], R // block_rows, K // FP8_BLOCK), dtype=np.int8)
    for i in range(s2.shape[0]):
        lib().orc_quantize_fp8(R, K, block_rows, _p(s2[i]), _p(q[i]), _p(e[i]))
    return q.reshape(*lead, R, K), e.reshape(*lead, R // block_rows, K // FP8_BLOCK)


def fp8_gemm(aq, ae, experts, wq, we, nthreads=0) -> np.ndarray:
    """Block-scaled GEMM: row i of codes aq [n,K] (exps ae [n,K/128]) against
    the weight rows of expert experts[i] (wq [E,N,K], we [E,N/128,K/128])."""
    aq, ae = _c(aq, np.uint8), _c(ae, np.int8)
    wq, we = _c(wq, np.uint8), _c(we, np.int8)
    experts = _c(experts, np.int32).reshape(-1)
    n, K = aq.shape
    N = wq.shape[1]
    y = np.empty((n, N), dtype=np.float32)
    rc = lib().orc_fp8_gemm(n, K, N, _p(aq), _p(ae), _p(experts), _p(wq), _p(we), _p(y), nthreads)
    if rc != 0:
        raise ValueError(f"orc_fp8_gemm rc={rc}")
    return y


def expert_ffn_fp8(tokens, experts, xq, xe, wgq, wge, wuq, wue, wdq, wde, nthreads=0,
                   want_act=False):
    tokens = _c(tokens, np.int32).reshape(-1)
    experts = _c(experts, np.int32).reshape(-1)
    n = tokens.size
    H = xq.shape[1]
    F = wgq.shape[1]
    args = [_c(a, np.uint8 if a.dtype == np.uint8 else np.int8)
            for a in (xq, xe, wgq, wge, wuq, wue, wdq, wde)]
    y = np.empty((n, H), dtype=np.float32)
    act = np.empty((n, F), dtype=np.uint16) if want_act else None
    rc = lib().orc_expert_ffn_fp8(n, _p(tokens), _p(experts), H, F, *[_p(a) for a in args],
                                  _p(y), _p(act), nthreads)
    if rc != 0:
        raise ValueError(f"orc_expert_ffn_fp8 rc={rc}")
    return (y, act) if want_act else y


def forward_tokens_fp8(tokens, x, wr, xq, xe, wq, k, score, renorm=True, bias=None,
                       nthreads=0):
    """The FP8 layer for chosen tokens. wq = dict of quantised expert weights
    (wgq, wge, wuq, wue, wdq, wde).  -> (out bf16 bits [n,H], ids, w)."""
    x, wr = _u16(x), _u16(wr)
    tokens = _c(tokens, np.int32).reshape(-1)
    n = tokens.size
    T, H = x.shape
    E, F = wq["wgq"].shape[0], wq["wgq"].shape[1]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((n, H), dtype=np.uint16)
    ids = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float32)
    rc = lib().orc_forward_tokens_fp8(n, _p(tokens), H, E, F, k, score, int(renorm), _p(x),
                                      _p(wr), _p(b), _p(_c(xq, np.uint8)), _p(_c(xe, np.int8)),
                                      *[_p(_c(wq[n_], np.uint8 if n_.endswith("q") else np.int8))
                                        for n_ in ("wgq", "wge", "wuq", "wue", "wdq", "wde")],
                                      _p(out), _p(ids), _p(w), nthreads)
    if rc != 0:
        raise ValueError(f"orc_forward_tokens_fp8 rc={rc}")
    return out, ids, w
