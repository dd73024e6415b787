"""The C ABI without a GPU: exported symbols, binding signatures and every
host-side argument check (all of which return before anything is enqueued)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from serve_router_gemm_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, ALIGN, UNSUP, WS, SCRATCH = 0, -1, -2, -3, -4, -5, -7


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        from serve_router_gemm_amd import build
        build.build(verbose=False)
    return M.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) >= {"moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine",
                          "moe_forward", "moe_expert_gate_up", "moe_expert_down",
                          "moe_workspace_bytes", "moe_status_string", "moe_version"}
    raw = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_binding_covers_header(L):
    assert sorted(M.SIGNATURES) == declared_functions()


def test_binding_arity_matches_header(L):
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, (_, args) in M.SIGNATURES.items():
        m = re.search(name + r"\s*\(([^)]*)\)", src)
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), name


def test_version_and_status_strings(L):
    assert L.moe_version() >= 10000
    for rc in (OK, NULL, SHAPE, ALIGN, UNSUP, WS, -6, SCRATCH):
        s = L.moe_status_string(rc).decode()
        assert s and s != "unknown status"
    assert L.moe_status_string(-99).decode() == "unknown status"


FAKE = ctypes.c_void_p(0x10000)     # aligned, never dereferenced: checks fail first
MIS = ctypes.c_void_p(0x10004)      # misaligned


def route(L, T=4, H=64, E=8, k=2, score=0, renorm=1, x=FAKE, wr=FAKE, b=None, ids=FAKE,
          w=FAKE, ws=FAKE, ws_bytes=0):
    return L.moe_route(T, H, E, k, score, renorm, x, wr, b, ids, w, ws, ws_bytes, None)


def test_route_checks(L):
    assert route(L, x=None) == NULL
    assert route(L, ws=None) == NULL
    assert route(L, E=0) == SHAPE
    assert route(L, E=513) == SHAPE
    assert route(L, k=9) == SHAPE          # k > E
    assert route(L, k=0) == SHAPE
    assert route(L, E=32, k=17) == SHAPE   # k > 16
    assert route(L, H=100) == UNSUP
    assert route(L, H=32) == SHAPE
    assert route(L, T=-1) == SHAPE
    assert route(L, T=(1 << 24) // 2 + 1) == SHAPE    # T*k > 2^24
    assert route(L, score=2) == UNSUP
    assert route(L, renorm=2) == UNSUP
    assert route(L, b=FAKE) == UNSUP       # bias with softmax
    assert route(L, x=MIS) == ALIGN
    assert route(L, score=1, b=MIS) == ALIGN
    assert route(L, ws_bytes=0) == WS
    assert route(L, T=0, x=None, wr=None, ids=None, w=None, ws=None) == OK


def test_permute_checks(L):
    p = L.moe_permute
    assert p(4, 8, 2, None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == NULL
    assert p(4, 8, 9, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == SHAPE
    assert p(4, 8, 2, FAKE, FAKE, MIS, FAKE, FAKE, FAKE, 0, None) == ALIGN
    # small batches (<= 16384 assignments) need no workspace; larger ones do
    assert L.moe_workspace_bytes(M.OP_PERMUTE, 2048, 64, 8, 64, 8, 0) == 0
    assert L.moe_workspace_bytes(M.OP_PERMUTE, 2049, 64, 8, 64, 8, 0) > 0
    assert p(2049, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == NULL
    assert p(2049, 8, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == WS
    assert p(0, 8, 2, None, None, None, None, None, None, 0, None) == OK


def test_gemm_checks(L):
    g = L.moe_expert_gate_up
    args = [FAKE] * 6
    assert g(4, 64, 8, 64, 2, *args, FAKE, 0, None) == WS
    assert g(4, 64, 8, 96, 2, *args, FAKE, 0, None) == UNSUP       # F % 64
    assert g(4, 64, 8, 64, 2, None, *args[1:], FAKE, 0, None) == NULL
    assert g(4, 64, 8, 64, 2, *args[:5], MIS, FAKE, 0, None) == ALIGN
    assert g(0, 64, 8, 64, 2, *([None] * 6), None, 0, None) == OK
    d = L.moe_expert_down
    assert d(4, 64, 8, 64, 2, *([FAKE] * 5), 0, FAKE, 0, None) == WS
    assert d(4, 64, 8, 64, 2, *([FAKE] * 5), 7, FAKE, 0, None) == UNSUP   # variant
    s = L.moe_grouped_swiglu
    assert s(4, 64, 8, 64, 2, *([FAKE] * 7), 0, FAKE, 0, None) == WS
    # T*k*max(H,F) must stay below 2^31
    assert s(1 << 16, 65536, 8, 64, 1, *([FAKE] * 7), 0, FAKE, 0, None) == SHAPE


def test_combine_and_forward_checks(L):
    c = L.moe_combine
    assert c(4, 64, 2, None, FAKE, FAKE, None) == NULL
    assert c(4, 64, 2, FAKE, FAKE, MIS, None) == ALIGN
    assert c(4, 65, 2, FAKE, FAKE, FAKE, None) == UNSUP
    assert c(0, 64, 2, None, None, None, None) == OK
    f = L.moe_forward
    base = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None]
    assert f(4, 64, 8, 64, 2, 0, 1, *base, 0, FAKE, 0, None) == WS
    assert f(4, 64, 8, 64, 2, 1, 1, *base, 0, FAKE, 0, None) == WS        # sigmoid, no bias
    b2 = list(base)
    b2[2] = FAKE
    assert f(4, 64, 8, 64, 2, 0, 1, *b2, 0, FAKE, 0, None) == UNSUP      # softmax + bias
    assert f(4, 64, 8, 64, 2, 0, 1, *base, 3, FAKE, 0, None) == UNSUP    # variant
    assert f(4, 64, 8, 64, 2, 0, 1, *base, 0, None, 0, None) == NULL
    b3 = list(base)
    b3[8] = MIS
    assert f(4, 64, 8, 64, 2, 0, 1, *b3, 0, FAKE, 0, None) == ALIGN
    assert f(0, 64, 8, 64, 2, 0, 1, *([None] * 9), 0, None, 0, None) == OK


def test_forward_static_checks(L):
    """moe_forward_static: moe_forward's checks, and sizes whose workspace
    exceeds the 32 MiB static scratch rejected before any HIP call."""
    f = L.moe_forward_static
    base = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None]
    b2 = list(base)
    b2[2] = FAKE
    assert f(4, 64, 8, 64, 2, 0, 1, *b2, 0, None) == UNSUP      # softmax + bias
    assert f(4, 64, 8, 64, 2, 0, 1, *base, 3, None) == UNSUP    # variant
    assert f(4, 64, 8, 96, 2, 0, 1, *base, 0, None) == UNSUP    # F % 64
    assert f(4, 64, 8, 64, 9, 0, 1, *base, 0, None) == SHAPE    # k > E
    b0 = list(base)
    b0[0] = None
    assert f(4, 64, 8, 64, 2, 0, 1, *b0, 0, None) == NULL
    b3 = list(base)
    b3[6] = MIS
    assert f(4, 64, 8, 64, 2, 0, 1, *b3, 0, None) == ALIGN
    assert f(0, 64, 8, 64, 2, 0, 1, *([None] * 9), 0, None) == OK
    # the decode layer (H 6144, E 256, F 2048, top-8) fits up to 132 tokens
    wb = L.moe_workspace_bytes
    assert wb(M.OP_FORWARD, 132, 6144, 256, 2048, 8, 0) <= 32 << 20
    assert wb(M.OP_FORWARD, 133, 6144, 256, 2048, 8, 0) > 32 << 20
    assert f(133, 6144, 256, 2048, 8, 1, 1, *base, 0, None) == SCRATCH
    assert f(16384, 6144, 256, 2048, 8, 1, 1, *base, 1, None) == SCRATCH


def test_workspace_sizes(L):
    wb = L.moe_workspace_bytes
    T, H, E, F, k = 16384, 6144, 256, 2048, 8
    fwd = wb(M.OP_FORWARD, T, H, E, F, k, 0)
    y = T * k * H * 4
    hact = T * k * F * 2
    assert fwd >= y + hact
    assert fwd < y + hact + (1 << 30)
    assert wb(M.OP_GROUPED_SWIGLU, T, H, E, F, k, 0) >= hact
    assert wb(M.OP_ROUTE, T, H, E, F, k, 0) >= T * E * 4
    assert wb(M.OP_PERMUTE, T, H, E, F, k, 0) >= E * 4
    assert wb(M.OP_COMBINE, T, H, E, F, k, 0) == 0
    # rejected sizes report 0
    assert wb(M.OP_FORWARD, T, 100, E, F, k, 0) == 0
    assert wb(M.OP_FORWARD, T, H, E, F, k, 5) == 0
    assert wb(99, T, H, E, F, k, 0) == 0


def test_decode_measurement_checks(L):
    lm = L.moe_lm_head_logits
    assert lm(4, 64, 100, None, FAKE, FAKE, None) == NULL
    assert lm(4, 64, 100, FAKE, MIS, FAKE, None) == ALIGN
    assert lm(4, 65, 100, FAKE, FAKE, FAKE, None) == UNSUP
    assert lm(4, 64, 0, FAKE, FAKE, FAKE, None) == SHAPE
    assert lm(4, 64, (1 << 20) + 1, FAKE, FAKE, FAKE, None) == SHAPE
    assert lm(-1, 64, 100, FAKE, FAKE, FAKE, None) == SHAPE
    assert lm(0, 64, 100, None, None, None, None) == OK
    ls = L.moe_log_softmax
    wb = L.moe_workspace_bytes
    need = wb(M.OP_LOG_SOFTMAX, 64, 65536, 1, 64, 1, 0)     # H carries V
    assert 64 * 256 * 4 <= need < 64 * 4096 * 4               # chunk sums and segment maxima
    assert ls(4, 100, None, FAKE, FAKE, 1 << 20, None) == NULL
    assert ls(4, 100, FAKE, FAKE, None, 1 << 20, None) == NULL
    assert ls(4, 100, FAKE, MIS, FAKE, 1 << 20, None) == ALIGN
    assert ls(4, 100, FAKE, FAKE, MIS, 1 << 20, None) == ALIGN
    assert ls(64, 65536, FAKE, FAKE, FAKE, need - 1, None) == WS
    assert ls(4, 0, FAKE, FAKE, FAKE, 0, None) == SHAPE
    assert ls(1 << 12, 1 << 20, FAKE, FAKE, FAKE, 0, None) == SHAPE       # T*V >= 2^31
    assert ls(0, 100, None, None, None, 0, None) == OK
    k3 = L.moe_k3
    need = wb(M.OP_K3, 64, 65536, 1, 64, 1, 0)
    assert need >= 64 * 256 * 8
    assert k3(4, 100, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == NULL
    assert k3(4, 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1 << 20, None) == NULL
    assert k3(4, 100, FAKE, FAKE, FAKE, MIS, FAKE, FAKE, 1 << 20, None) == ALIGN
    assert k3(64, 65536, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WS
    assert k3(4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == SHAPE
    assert k3(0, 100, None, None, None, None, None, None, 0, None) == OK
    assert wb(M.OP_K3, 4, 0, 1, 64, 1, 0) == 0


def test_forward_replay_checks(L):
    f = L.moe_forward_replay
    # T, H, E, F, k, score, renorm, x, w_router, ids, w, wg, wu, wd, out, w_out, variant, ws, bytes
    def call(T=4, H=64, E=8, F=64, k=2, score=0, renorm=1, x=FAKE, wr=FAKE, ids=FAKE, w=None,
             wg=FAKE, wu=FAKE, wd=FAKE, out=FAKE, w_out=None, variant=0, ws=FAKE, nbytes=1 << 40):
        return f(T, H, E, F, k, score, renorm, x, wr, ids, w, wg, wu, wd, out, w_out, variant,
                 ws, nbytes, None)
    assert call(ids=None) == NULL
    assert call(wr=None, w=None) == NULL            # weights neither given nor computable
    assert call(wr=None, w=FAKE, nbytes=0) == WS     # recorded weights: no router needed
    assert call(w_out=MIS) == ALIGN
    assert call(H=65) == UNSUP
    assert call(score=3) == UNSUP
    assert call(variant=2) == UNSUP
    assert call(k=9) == SHAPE
    assert call(nbytes=0) == WS
    assert call(T=0, x=None, wr=None, ids=None, wg=None, wu=None, wd=None, out=None, ws=None) == OK


def test_topk_large_checks(L):
    t = L.moe_topk_large
    assert t(-1, 100, 10, FAKE, None, FAKE, None, None) == SHAPE
    assert t(4, 0, 10, FAKE, None, FAKE, None, None) == SHAPE
    assert t(4, 100, 0, FAKE, None, FAKE, None, None) == SHAPE
    assert t(4, 100, 4097, FAKE, None, FAKE, None, None) == SHAPE
    assert t(4, (1 << 24) + 1, 10, FAKE, None, FAKE, None, None) == SHAPE
    assert t(1 << 8, 1 << 24, 10, FAKE, None, FAKE, None, None) == SHAPE     # Q*N >= 2^31
    assert t(4, 100, 10, None, None, FAKE, None, None) == NULL
    assert t(4, 100, 10, FAKE, None, None, None, None) == NULL
    assert t(4, 100, 10, FAKE, MIS, FAKE, None, None) == ALIGN
    assert t(4, 100, 10, FAKE, None, FAKE, MIS, None) == ALIGN
    assert t(0, 100, 10, None, None, None, None, None) == OK


def test_fp8_checks(L):
    q = L.moe_quantize_fp8
    assert q(-1, 256, 1, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(4, 192, 1, FAKE, FAKE, FAKE, None) == SHAPE           # K not in 128-blocks
    assert q(4, 0, 1, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(4, 256, 0, FAKE, FAKE, FAKE, None) == SHAPE
    assert q(6, 256, 4, FAKE, FAKE, FAKE, None) == SHAPE           # R % block_rows
    assert q(1 << 26, 1 << 15, 1, FAKE, FAKE, FAKE, None) == SHAPE  # R*K > 2^40
    assert q(4, 256, 1, None, FAKE, FAKE, None) == NULL
    assert q(4, 256, 1, FAKE, FAKE, MIS, None) == ALIGN
    assert q(0, 256, 1, None, None, None, None) == OK
    gu = L.moe_expert_gate_up_fp8
    # T, H, E, F, k, xq, xe, perm, offs, wg_q, wg_e, wu_q, wu_e, aq, ae, ab, ws, bytes
    def call_gu(T=4, H=256, E=8, F=256, k=2, xq=FAKE, ab=None, ws=FAKE, nbytes=1 << 20):
        return gu(T, H, E, F, k, xq, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ab,
                  ws, nbytes, None)
    assert call_gu(H=192) == UNSUP                                  # 64-multiple, not 128
    assert call_gu(F=320) == UNSUP
    assert call_gu(H=8192 + 128) == SHAPE                           # K side > 8192
    assert call_gu(xq=None) == NULL
    assert call_gu(ab=MIS) == ALIGN
    assert call_gu(nbytes=0) == WS
    assert call_gu(T=0, xq=None, ws=None) == OK
    dn = L.moe_expert_down_fp8
    assert dn(4, 256, 8, 8192 + 128, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
              None) == SHAPE                                        # F is the K side here
    assert dn(4, 256, 8, 256, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == WS
    assert dn(4, 256, 8, 256, 2, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
              None) == NULL
    f = L.moe_forward_fp8
    def call_f(T=4, H=256, E=8, F=256, k=2, score=0, bias=None, x=FAKE, nbytes=1 << 40):
        return f(T, H, E, F, k, score, 1, x, FAKE, bias, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                 FAKE, None, None, FAKE, nbytes, None)
    assert call_f(score=0, bias=FAKE) == UNSUP
    assert call_f(score=2) == UNSUP
    assert call_f(x=None) == NULL
    assert call_f(nbytes=0) == WS
    assert call_f(H=192) == UNSUP
    assert call_f(T=0, x=None) == OK
    wb = L.moe_workspace_bytes
    T, H, E, F, k = 16384, 6144, 256, 2048, 8
    A = T * k
    fwd8 = wb(M.OP_FORWARD_FP8, T, H, E, F, k, 0)
    assert fwd8 >= A * H * 4 + A * F + T * H
    assert fwd8 < wb(M.OP_FORWARD, T, H, E, F, k, 0)               # fp8 act is half the bytes
    assert wb(M.OP_GATE_UP_FP8, T, H, E, F, k, 0) == wb(M.OP_GATE_UP, T, H, E, F, k, 0)
    assert wb(M.OP_DOWN_FP8, T, H, E, F, k, 1) == 0                 # no split-K FP8 variant
    assert wb(M.OP_FORWARD_FP8, T, 192, E, F, k, 0) == 0
