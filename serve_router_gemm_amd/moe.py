"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function takes torch tensors on the ROCm device, checks dtypes and
shapes, allocates outputs and workspace with torch (device memory is torch's
job here), and calls the C entry point of the same name on torch's current
stream.  No step of the layer runs in Python or torch: if libmoe.so is
missing, importing the library raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
INVARIANT = 0
SPLITK_VARIANT = 1

(OP_ROUTE, OP_PERMUTE, OP_GATE_UP, OP_DOWN, OP_GROUPED_SWIGLU, OP_COMBINE, OP_FORWARD,
 OP_GATE_UP_FP8, OP_DOWN_FP8, OP_FORWARD_FP8, OP_LOG_SOFTMAX, OP_K3) = range(12)
FP8_BLOCK = 128

STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
          -4: "MOE_ERR_UNSUPPORTED", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP",
          -7: "MOE_ERR_SCRATCH"}

# name -> (restype, argtypes); must match include/moe.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
SIGNATURES = {
    "moe_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_version": (_I, []),
    "moe_route": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_permute": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_gate_up": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_down": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "moe_grouped_swiglu": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _Z,
                                _P]),
    "moe_combine": (_I, [_I, _I, _I, _P, _P, _P, _P]),
    "moe_forward": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                         _P, _Z, _P]),
    "moe_forward_static": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _I, _P]),
    "moe_forward_replay": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _I, _P, _Z, _P]),
    "moe_topk_large": (_I, [_I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_lm_head_logits": (_I, [_I, _I, _I, _P, _P, _P, _P]),
    "moe_log_softmax": (_I, [_I, _I, _P, _P, _P, _Z, _P]),
    "moe_k3": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_quantize_fp8": (_I, [_I, _I, _I, _P, _P, _P, _P]),
    "moe_expert_gate_up_fp8": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _Z, _P]),
    "moe_expert_down_fp8": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_forward_fp8": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _P, _P, _P, _Z, _P]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        self.rc = rc
        msg = lib().moe_status_string(rc).decode()
        super().__init__(f"{fn} returned {STATUS.get(rc, rc)}: {msg}")


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m serve_router_gemm_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc)


def workspace_bytes(op, T, H, E, F, top_k, variant=INVARIANT) -> int:
    return int(lib().moe_workspace_bytes(op, T, H, E, F, top_k, variant))


def workspace(op, T, H, E, F, top_k, variant=INVARIANT, device="cuda"):
    n = workspace_bytes(op, T, H, E, F, top_k, variant)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ws(ws, need, device):
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _dev(ws, "ws", torch.uint8)
    return ws


def route(x, w_router, top_k, score=SCORE_SOFTMAX, renormalize=True, bias=None,
          topk_ids=None, topk_w=None, ws=None, stream=None):
    """moe_route: -> (topk_ids [T,k] int32, topk_w [T,k] fp32)."""
    T, H = x.shape
    E = w_router.shape[0]
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, H))
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    ids = topk_ids if topk_ids is not None else torch.empty((T, top_k), dtype=torch.int32,
                                                             device=x.device)
    w = topk_w if topk_w is not None else torch.empty((T, top_k), dtype=torch.float32,
                                                       device=x.device)
    _dev(ids, "topk_ids", torch.int32, (T, top_k))
    _dev(w, "topk_w", torch.float32, (T, top_k))
    need = workspace_bytes(OP_ROUTE, T, H, E, 64, top_k)
    ws = _ws(ws, need, x.device)
    rc = lib().moe_route(T, H, E, top_k, int(score), int(bool(renormalize)), _ptr(x),
                         _ptr(w_router), _ptr(bias), _ptr(ids), _ptr(w), _ptr(ws), ws.numel(),
                         _stream(stream))
    _check("moe_route", rc)
    return ids, w


def permute(topk_ids, E, counts=None, offsets=None, perm=None, inv_perm=None, ws=None,
            stream=None):
    """moe_permute: -> (counts [E], offsets [E+1], perm [A], inv_perm [A]) int32."""
    T, k = topk_ids.shape
    _dev(topk_ids, "topk_ids", torch.int32)
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(T * k, dtype=torch.int32, device=dev) if perm is None else perm
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if inv_perm is None else inv_perm
    _dev(counts, "expert_counts", torch.int32, (E,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(perm, "perm", torch.int32, (T * k,))
    _dev(inv, "inv_perm", torch.int32, (T * k,))
    ws = _ws(ws, workspace_bytes(OP_PERMUTE, T, 64, E, 64, k), dev)
    rc = lib().moe_permute(T, E, k, _ptr(topk_ids), _ptr(counts), _ptr(offsets), _ptr(perm),
                           _ptr(inv), _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_permute", rc)
    return counts, offsets, perm, inv


def expert_gate_up(x, perm, offsets, w_gate, w_up, top_k, h_act=None, ws=None, stream=None):
    """moe_expert_gate_up: -> h_act [T*k, F] bf16 (rows in permuted order)."""
    T, H = x.shape
    E, F = w_gate.shape[0], w_gate.shape[1]
    _dev(x, "x", torch.bfloat16)
    _dev(perm, "perm", torch.int32, (T * top_k,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(w_gate, "w_gate", torch.bfloat16, (E, F, H))
    _dev(w_up, "w_up", torch.bfloat16, (E, F, H))
    if h_act is None:
        h_act = torch.empty((T * top_k, F), dtype=torch.bfloat16, device=x.device)
    _dev(h_act, "h_act", torch.bfloat16, (T * top_k, F))
    ws = _ws(ws, workspace_bytes(OP_GATE_UP, T, H, E, F, top_k), x.device)
    rc = lib().moe_expert_gate_up(T, H, E, F, top_k, _ptr(x), _ptr(perm), _ptr(offsets),
                                  _ptr(w_gate), _ptr(w_up), _ptr(h_act), _ptr(ws), ws.numel(),
                                  _stream(stream))
    _check("moe_expert_gate_up", rc)
    return h_act


def expert_down(h_act, perm, offsets, w_down, top_k, variant=INVARIANT, y=None, ws=None,
                stream=None):
    """moe_expert_down: -> y [T*k, H] fp32 (rows in assignment order)."""
    A, F = h_act.shape
    E, H = w_down.shape[0], w_down.shape[1]
    T = A // top_k
    _dev(h_act, "h_act", torch.bfloat16)
    _dev(perm, "perm", torch.int32, (A,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(w_down, "w_down", torch.bfloat16, (E, H, F))
    if y is None:
        y = torch.empty((A, H), dtype=torch.float32, device=h_act.device)
    _dev(y, "y", torch.float32, (A, H))
    ws = _ws(ws, workspace_bytes(OP_DOWN, T, H, E, F, top_k, variant), h_act.device)
    rc = lib().moe_expert_down(T, H, E, F, top_k, _ptr(h_act), _ptr(perm), _ptr(offsets),
                               _ptr(w_down), _ptr(y), int(variant), _ptr(ws), ws.numel(),
                               _stream(stream))
    _check("moe_expert_down", rc)
    return y


def grouped_swiglu(x, perm, offsets, w_gate, w_up, w_down, top_k, variant=INVARIANT, y=None,
                   ws=None, stream=None):
    """moe_grouped_swiglu: both expert GEMMs -> y [T*k, H] fp32."""
    T, H = x.shape
    E, F = w_gate.shape[0], w_gate.shape[1]
    _dev(x, "x", torch.bfloat16)
    _dev(perm, "perm", torch.int32, (T * top_k,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(w_gate, "w_gate", torch.bfloat16, (E, F, H))
    _dev(w_up, "w_up", torch.bfloat16, (E, F, H))
    _dev(w_down, "w_down", torch.bfloat16, (E, H, F))
    if y is None:
        y = torch.empty((T * top_k, H), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32, (T * top_k, H))
    ws = _ws(ws, workspace_bytes(OP_GROUPED_SWIGLU, T, H, E, F, top_k, variant), x.device)
    rc = lib().moe_grouped_swiglu(T, H, E, F, top_k, _ptr(x), _ptr(perm), _ptr(offsets),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), int(variant),
                                  _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_grouped_swiglu", rc)
    return y


def combine(y, topk_w, out=None, stream=None):
    """moe_combine: -> out [T, H] bf16."""
    T, k = topk_w.shape
    A, H = y.shape
    _dev(y, "y", torch.float32, (T * k, H))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _dev(out, "out", torch.bfloat16, (T, H))
    rc = lib().moe_combine(T, H, k, _ptr(y), _ptr(topk_w), _ptr(out), _stream(stream))
    _check("moe_combine", rc)
    return out


def forward(x, w_router, w_gate, w_up, w_down, top_k, score=SCORE_SOFTMAX, renormalize=True,
            bias=None, variant=INVARIANT, out=None, topk_ids=None, topk_w=None, ws=None,
            stream=None, return_routing=False):
    """moe_forward: the whole layer -> out [T, H] bf16 (and routing if asked)."""
    T, H = x.shape
    E, F = w_gate.shape[0], w_gate.shape[1]
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, H))
    _dev(w_gate, "w_gate", torch.bfloat16, (E, F, H))
    _dev(w_up, "w_up", torch.bfloat16, (E, F, H))
    _dev(w_down, "w_down", torch.bfloat16, (E, H, F))
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev(out, "out", torch.bfloat16, (T, H))
    if return_routing:
        if topk_ids is None:
            topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        if topk_w is None:
            topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    if topk_ids is not None:
        _dev(topk_ids, "topk_ids", torch.int32, (T, top_k))
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, (T, top_k))
    ws = _ws(ws, workspace_bytes(OP_FORWARD, T, H, E, F, top_k, variant), dev)
    rc = lib().moe_forward(T, H, E, F, top_k, int(score), int(bool(renormalize)), _ptr(x),
                           _ptr(w_router), _ptr(bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                           _ptr(out), _ptr(topk_ids), _ptr(topk_w), int(variant), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check("moe_forward", rc)
    if return_routing:
        return out, topk_ids, topk_w
    return out


def forward_static(x, w_router, w_gate, w_up, w_down, top_k, score=SCORE_SOFTMAX,
                   renormalize=True, bias=None, variant=INVARIANT, out=None, topk_ids=None,
                   topk_w=None, stream=None):
    """moe_forward_static: moe_forward with the library's static per-GPU scratch
    instead of a workspace (nothing is allocated by the call itself; `out` and
    the routing outputs must then be passed in)."""
    T, H = x.shape
    E, F = w_gate.shape[0], w_gate.shape[1]
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, H))
    _dev(w_gate, "w_gate", torch.bfloat16, (E, F, H))
    _dev(w_up, "w_up", torch.bfloat16, (E, F, H))
    _dev(w_down, "w_down", torch.bfloat16, (E, H, F))
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, (T, H))
    if topk_ids is not None:
        _dev(topk_ids, "topk_ids", torch.int32, (T, top_k))
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, (T, top_k))
    rc = lib().moe_forward_static(T, H, E, F, top_k, int(score), int(bool(renormalize)),
                                  _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate), _ptr(w_up),
                                  _ptr(w_down), _ptr(out), _ptr(topk_ids), _ptr(topk_w),
                                  int(variant), _stream(stream))
    _check("moe_forward_static", rc)
    return out


def forward_replay(x, topk_ids, w_gate, w_up, w_down, topk_w=None, w_router=None,
                   score=SCORE_SOFTMAX, renormalize=True, variant=INVARIANT, ws=None,
                   stream=None, return_weights=False):
    """moe_forward_replay: the layer with recorded experts (router replay).

    topk_w=None recomputes the weights from w_router for the given experts;
    return_weights=True then also returns them."""
    T, H = x.shape
    E, F, _ = w_gate.shape
    k = topk_ids.shape[1]
    _dev(x, "x", torch.bfloat16, (T, H))
    _dev(topk_ids, "topk_ids", torch.int32, (T, k))
    _dev(w_gate, "w_gate", torch.bfloat16, (E, F, H))
    _dev(w_up, "w_up", torch.bfloat16, (E, F, H))
    _dev(w_down, "w_down", torch.bfloat16, (E, H, F))
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, (T, k))
    if w_router is not None:
        _dev(w_router, "w_router", torch.bfloat16, (E, H))
    out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    w_out = None
    if topk_w is None and return_weights:
        w_out = torch.empty((T, k), dtype=torch.float32, device=x.device)
    need = workspace_bytes(OP_FORWARD, T, H, E, F, k, variant)
    ws = _ws(ws, need, x.device)
    rc = lib().moe_forward_replay(T, H, E, F, k, score, int(renormalize), _ptr(x),
                                  _ptr(w_router), _ptr(topk_ids), _ptr(topk_w), _ptr(w_gate),
                                  _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(w_out), variant,
                                  _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_forward_replay", rc)
    return (out, w_out) if return_weights else out


def lm_head_logits(h, proj, z=None, stream=None):
    """moe_lm_head_logits: z [T, V] fp32 = h [T, H] . proj [V, H]^T in the pinned order."""
    T, H = h.shape
    V = proj.shape[0]
    _dev(h, "h", torch.bfloat16, (T, H))
    _dev(proj, "proj", torch.bfloat16, (V, H))
    if z is None:
        z = torch.empty((T, V), dtype=torch.float32, device=h.device)
    _dev(z, "z", torch.float32, (T, V))
    rc = lib().moe_lm_head_logits(T, H, V, _ptr(h), _ptr(proj), _ptr(z), _stream(stream))
    _check("moe_lm_head_logits", rc)
    return z


def log_softmax(z, out=None, ws=None, stream=None):
    """moe_log_softmax: fp32 log-softmax over the last axis (out may be z)."""
    T, V = z.shape
    _dev(z, "z", torch.float32, (T, V))
    if out is None:
        out = torch.empty_like(z)
    _dev(out, "out", torch.float32, (T, V))
    ws = _ws(ws, workspace_bytes(OP_LOG_SOFTMAX, T, V, 1, 64, 1), z.device)
    rc = lib().moe_log_softmax(T, V, _ptr(z), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_log_softmax", rc)
    return out


def k3(logp_ref, logp_test, ws=None, stream=None):
    """moe_k3: -> (k3_mean [T] fp64, k3_greedy [T] fp64, greedy [T] int32)."""
    T, V = logp_test.shape
    _dev(logp_ref, "logp_ref", torch.float32, (T, V))
    _dev(logp_test, "logp_test", torch.float32, (T, V))
    dev = logp_test.device
    mean = torch.empty(T, dtype=torch.float64, device=dev)
    gk3 = torch.empty(T, dtype=torch.float64, device=dev)
    g = torch.empty(T, dtype=torch.int32, device=dev)
    ws = _ws(ws, workspace_bytes(OP_K3, T, V, 1, 64, 1), dev)
    rc = lib().moe_k3(T, V, _ptr(logp_ref), _ptr(logp_test), _ptr(mean), _ptr(gk3), _ptr(g),
                      _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_k3", rc)
    return mean, gk3, g


def topk_large(scores, k, lengths=None, want_vals=True, stream=None):
    """moe_topk_large: -> (idx [Q,k] int32, vals [Q,k] fp32 or None)."""
    Q, N = scores.shape
    _dev(scores, "scores", torch.float32, (Q, N))
    if lengths is not None:
        _dev(lengths, "lengths", torch.int32, (Q,))
    idx = torch.empty((Q, k), dtype=torch.int32, device=scores.device)
    vals = torch.empty((Q, k), dtype=torch.float32, device=scores.device) if want_vals else None
    rc = lib().moe_topk_large(Q, N, k, _ptr(scores), _ptr(lengths), _ptr(idx), _ptr(vals),
                              _stream(stream))
    _check("moe_topk_large", rc)
    return idx, vals



# ---------------------------------------------------------------------------
# FP8 rollout path
# ---------------------------------------------------------------------------
def quantize_fp8(src, block_rows, q=None, e=None, stream=None):
    """moe_quantize_fp8: bf16 [..., R, K] -> (codes uint8 [..., R, K], exps int8
    [..., R/block_rows, K/128]); the leading axes fold into rows (blocks never
    cross them when R % block_rows == 0)."""
    _dev(src, "src", torch.bfloat16)
    *lead, R, K = src.shape
    if R % block_rows:
        raise ValueError("R must be a multiple of block_rows")
    rows = src.numel() // K if src.numel() else 0
    if q is None:
        q = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    if e is None:
        e = torch.empty((*lead, R // block_rows, K // FP8_BLOCK), dtype=torch.int8,
                        device=src.device)
    _dev(q, "q", torch.uint8, src.shape)
    _dev(e, "exps", torch.int8, (*lead, R // block_rows, K // FP8_BLOCK))
    rc = lib().moe_quantize_fp8(rows, K, block_rows, _ptr(src), _ptr(q), _ptr(e),
                                _stream(stream))
    _check("moe_quantize_fp8", rc)
    return q, e


def quantize_weights_fp8(w_gate, w_up, w_down, stream=None) -> dict:
    """The three expert weight tensors in 128 x 128 blocks -> dict of
    wg_q, wg_e, wu_q, wu_e, wd_q, wd_e."""
    wq = {}
    wq["wg_q"], wq["wg_e"] = quantize_fp8(w_gate, FP8_BLOCK, stream=stream)
    wq["wu_q"], wq["wu_e"] = quantize_fp8(w_up, FP8_BLOCK, stream=stream)
    wq["wd_q"], wq["wd_e"] = quantize_fp8(w_down, FP8_BLOCK, stream=stream)
    return wq


def _check_wq(wq, E, F, H):
    _dev(wq["wg_q"], "wg_q", torch.uint8, (E, F, H))
    _dev(wq["wu_q"], "wu_q", torch.uint8, (E, F, H))
    _dev(wq["wd_q"], "wd_q", torch.uint8, (E, H, F))
    _dev(wq["wg_e"], "wg_e", torch.int8, (E, F // FP8_BLOCK, H // FP8_BLOCK))
    _dev(wq["wu_e"], "wu_e", torch.int8, (E, F // FP8_BLOCK, H // FP8_BLOCK))
    _dev(wq["wd_e"], "wd_e", torch.int8, (E, H // FP8_BLOCK, F // FP8_BLOCK))


def expert_gate_up_fp8(xq, xe, perm, offsets, wg_q, wg_e, wu_q, wu_e, top_k, want_bf16=False,
                       act_q=None, act_e=None, ws=None, stream=None):
    """moe_expert_gate_up_fp8: -> (act_q [T*k,F] uint8, act_e [T*k,F/128] int8,
    act bf16 [T*k,F] or None), rows in permuted order."""
    T, H = xq.shape
    E, F = wg_q.shape[0], wg_q.shape[1]
    _dev(xq, "xq", torch.uint8)
    _dev(xe, "xe", torch.int8, (T, H // FP8_BLOCK))
    _dev(perm, "perm", torch.int32, (T * top_k,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(wg_q, "wg_q", torch.uint8, (E, F, H))
    _dev(wu_q, "wu_q", torch.uint8, (E, F, H))
    _dev(wg_e, "wg_e", torch.int8, (E, F // FP8_BLOCK, H // FP8_BLOCK))
    _dev(wu_e, "wu_e", torch.int8, (E, F // FP8_BLOCK, H // FP8_BLOCK))
    dev = xq.device
    aq = torch.empty((T * top_k, F), dtype=torch.uint8, device=dev) if act_q is None else act_q
    ae = torch.empty((T * top_k, F // FP8_BLOCK), dtype=torch.int8, device=dev) \
        if act_e is None else act_e
    _dev(aq, "act_q", torch.uint8, (T * top_k, F))
    _dev(ae, "act_e", torch.int8, (T * top_k, F // FP8_BLOCK))
    ab = torch.empty((T * top_k, F), dtype=torch.bfloat16, device=dev) if want_bf16 else None
    ws = _ws(ws, workspace_bytes(OP_GATE_UP_FP8, T, H, E, F, top_k), dev)
    rc = lib().moe_expert_gate_up_fp8(T, H, E, F, top_k, _ptr(xq), _ptr(xe), _ptr(perm),
                                      _ptr(offsets), _ptr(wg_q), _ptr(wg_e), _ptr(wu_q),
                                      _ptr(wu_e), _ptr(aq), _ptr(ae), _ptr(ab), _ptr(ws),
                                      ws.numel(), _stream(stream))
    _check("moe_expert_gate_up_fp8", rc)
    return aq, ae, ab


def expert_down_fp8(act_q, act_e, perm, offsets, wd_q, wd_e, top_k, y=None, ws=None,
                    stream=None):
    """moe_expert_down_fp8: -> y [T*k, H] fp32 (rows in assignment order)."""
    A, F = act_q.shape
    E, H = wd_q.shape[0], wd_q.shape[1]
    T = A // top_k
    _dev(act_q, "act_q", torch.uint8)
    _dev(act_e, "act_e", torch.int8, (A, F // FP8_BLOCK))
    _dev(perm, "perm", torch.int32, (A,))
    _dev(offsets, "expert_offsets", torch.int32, (E + 1,))
    _dev(wd_q, "wd_q", torch.uint8, (E, H, F))
    _dev(wd_e, "wd_e", torch.int8, (E, H // FP8_BLOCK, F // FP8_BLOCK))
    if y is None:
        y = torch.empty((A, H), dtype=torch.float32, device=act_q.device)
    _dev(y, "y", torch.float32, (A, H))
    ws = _ws(ws, workspace_bytes(OP_DOWN_FP8, T, H, E, F, top_k), act_q.device)
    rc = lib().moe_expert_down_fp8(T, H, E, F, top_k, _ptr(act_q), _ptr(act_e), _ptr(perm),
                                   _ptr(offsets), _ptr(wd_q), _ptr(wd_e), _ptr(y), _ptr(ws),
                                   ws.numel(), _stream(stream))
    _check("moe_expert_down_fp8", rc)
    return y


def forward_fp8(x, w_router, wq, top_k, score=SCORE_SOFTMAX, renormalize=True, bias=None,
                out=None, ws=None, stream=None, return_routing=False):
    """moe_forward_fp8: the FP8 layer -> out [T, H] bf16 (and routing if asked).
    wq: the dict of quantize_weights_fp8."""
    T, H = x.shape
    E, F = wq["wg_q"].shape[0], wq["wg_q"].shape[1]
    _dev(x, "x", torch.bfloat16)
    _dev(w_router, "w_router", torch.bfloat16, (E, H))
    _check_wq(wq, E, F, H)
    if bias is not None:
        _dev(bias, "bias", torch.float32, (E,))
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev(out, "out", torch.bfloat16, (T, H))
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if return_routing else None
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if return_routing else None
    ws = _ws(ws, workspace_bytes(OP_FORWARD_FP8, T, H, E, F, top_k), dev)
    rc = lib().moe_forward_fp8(T, H, E, F, top_k, int(score), int(bool(renormalize)), _ptr(x),
                               _ptr(w_router), _ptr(bias), _ptr(wq["wg_q"]), _ptr(wq["wg_e"]),
                               _ptr(wq["wu_q"]), _ptr(wq["wu_e"]), _ptr(wq["wd_q"]),
                               _ptr(wq["wd_e"]), _ptr(out), _ptr(ids), _ptr(w), _ptr(ws),
                               ws.numel(), _stream(stream))
    _check("moe_forward_fp8", rc)
    return (out, ids, w) if return_routing else out
