#!/usr/bin/env python3
"""Benchmark of the batch-invariant MoE layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload large|mid|tie|dec|tiny]

One step is one pass of the whole path (route, permute, gate/up + SwiGLU,
down, combine) over one synthetic batch that is already resident in HBM.  The
step is enqueued as the five C entry points that moe_forward chains (checked
bitwise against moe_forward before timing), so HIP events on the launch stream
can time each stage inside the timed region.

Prints one JSON line: tokens/s, the dominant kernel's roofline fraction, the
oracle's CPU baseline on a bounded sample (at every host thread and at one),
parity of that sample against the GPU's output (id mismatches, near-tie
exemptions, largest error), the batch-invariance check of 16 probe tokens
(differing bits against each probe alone; must be 0), and the same step with
the load-dependent variant of both expert GEMMs (its time relative to the
invariant step, the outputs and probe bits it moves).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "MoE-layer tokens/s + MFMA util; bitwise-identical output across batch sizes"

# HBM bytes per launch of the gate/up kernel from rocprofv3 FETCH_SIZE (x2.0) and
# WRITE_SIZE (x1.0) on the large workload (profiles/expert_gemm_large_T16384.md),
# valid only for the sources and build flags they were taken on (gemm_source_hash).
TRAFFIC = {"kernel_sha256_prefix": "b93e4893faffabf1", "workload": "large", "bytes": 21.78e9}
GEMM_SOURCES = ("moe_gemm.hip", "moe_gemm_tiles.h", "moe_device.h", "moe_internal.h")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_FP32_VALU_TFLOPS = 78.6  # 256 CU x 64 lanes x 2 flop x 2.4 GHz, fp32 fma without packed math
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix peak


def route_uses_matrix_cores(T, H, E):
    """The router-logits kernel the library's route plan picks (route_plan in
    csrc/moe_route.hip): the K=1 fp32 MFMA kernel (32 x 64 per wave, blocks of
    2 x 2 waves for E > 64, else 4 x 1) when its folded tiles give 512 blocks,
    or, for 512 tokens or more, its one-block-per-chunk tiles give 256."""
    we = 2 if E > 64 else 1
    wt = 4 // we
    nchunks = (H + 255) // 256
    mb = ((T + 32 * wt - 1) // (32 * wt)) * ((E + 64 * we - 1) // (64 * we))
    return mb >= 512 or (T >= 512 and mb * nchunks >= 256)
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=["large", "mid", "tie", "dec", "tiny"])
    ap.add_argument("--T", type=int, default=None, help="override the workload's token count")
    ap.add_argument("--variant", type=int, default=0,
                    help="0 invariant, 1 the load-dependent variant")
    ap.add_argument("--cpu-sample", type=int, default=None,
                    help="tokens of the oracle CPU baseline (0 disables)")
    ap.add_argument("--no-check", action="store_true", help="skip the probe invariance check")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step and stop: no variant, replay, top-k, FP8 or decode "
                         "legs (short profiler runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (HBM counter calibration)")
    ap.add_argument("--print-gemm-hash", action="store_true",
                    help="print the hash of the GEMM sources and build flags, and exit")
    return ap.parse_args()


def gemm_source_hash():
    """sha256 of every source the expert GEMM kernels are compiled from, and of
    the build flags."""
    import hashlib
    from serve_router_gemm_amd import build as B
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(HERE, "serve_router_gemm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    h.update(" ".join(B.flags()).encode())
    return h.hexdigest()


def traffic_bytes(workload, T):
    """Profiled HBM bytes per gate/up launch, or None if a GEMM source or the
    build flags have changed since the counters were taken (or for another
    workload)."""
    if (TRAFFIC["bytes"] is None or not gemm_source_hash().startswith(TRAFFIC["kernel_sha256_prefix"])
            or workload != TRAFFIC["workload"] or T != 16384):
        return None
    return TRAFFIC["bytes"]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def calibrate_copy(mib):
    """Three device-to-device copies of a known size: the reference that the
    FETCH_SIZE / WRITE_SIZE counters are scaled against."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)


def main():
    args = parse()
    if args.print_gemm_hash:
        print(gemm_source_hash())
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the MoE layer runs on one GPU only (the layer forward on one "
              "MI355X); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from serve_router_gemm_amd import inputs as I
    from serve_router_gemm_amd import moe as M

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    M.lib()   # fail loudly if libmoe.so is missing
    dev = "cuda"

    cfg = I.CONFIGS[args.workload]
    if args.T is not None:
        cfg = I.scaled(cfg, T=args.T)
    T, H, E, F, k = cfg.T, cfg.H, cfg.E, cfg.F, cfg.k
    A = T * k
    log(f"[bench] workload {I.describe(cfg)}")
    t0 = time.time()
    L = I.make_layer(cfg, dev)
    n_probe = min(16, T)
    if cfg.name == "tie":
        # the near-tie construction: router rows and tokens with exactly known
        # logits (25% exact k-th/(k+1)-th ties, 25% one fp32 ulp apart); the
        # probes are 16 of its rows, stress tokens among them, each compared
        # with itself alone
        d = I.make_tie_inputs(cfg, T=T)
        L["w_router"] = d["w_router"].to(dev)
        x = d["x"].to(dev)
        probe_pos = list(np.sort(np.random.default_rng(3).choice(T, n_probe, replace=False)))
        probes = x[torch.tensor(probe_pos, device=dev)].contiguous()
    else:
        probes = I.probes(H, 16, dev)
        if T >= 16:
            x, probe_pos = I.embed_probes(probes, T, rep=0)
        else:
            # a batch smaller than the 16 probes: the batch is the first T probes
            x = probes[:T].contiguous()
            probe_pos = list(range(T))
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    bias = L["bias"]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(A, dtype=torch.int32, device=dev)
    inv = torch.empty(A, dtype=torch.int32, device=dev)
    h_act = torch.empty((A, F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((A, H), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws_r = M.workspace(M.OP_ROUTE, T, H, E, F, k)
    ws_p = M.workspace(M.OP_PERMUTE, T, H, E, F, k)
    ws_g = M.workspace(M.OP_GATE_UP, T, H, E, F, k)
    ws_d = M.workspace(M.OP_DOWN, T, H, E, F, k)
    ws_sv1 = M.workspace(M.OP_GROUPED_SWIGLU, T, H, E, F, k, 1) if args.variant else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        M.route(x, L["w_router"], k, cfg.score, cfg.renorm, bias=bias, topk_ids=ids, topk_w=w,
                ws=ws_r)
        if ev is not None:
            ev[1].record(stream)
        M.permute(ids, E, counts, offsets, perm, inv, ws=ws_p)
        if ev is not None:
            ev[2].record(stream)
        if args.variant:
            # the load-dependent variant of both GEMMs (one stage here)
            M.grouped_swiglu(x, perm, offsets, L["w_gate"], L["w_up"], L["w_down"], k,
                             variant=1, y=y, ws=ws_sv1)
            if ev is not None:
                ev[3].record(stream)
                ev[4].record(stream)
        else:
            M.expert_gate_up(x, perm, offsets, L["w_gate"], L["w_up"], k, h_act=h_act, ws=ws_g)
            if ev is not None:
                ev[3].record(stream)
            M.expert_down(h_act, perm, offsets, L["w_down"], k, y=y, ws=ws_d)
            if ev is not None:
                ev[4].record(stream)
        M.combine(y, w, out=out)
        if ev is not None:
            ev[5].record(stream)

    # the staged step is moe_forward: check once, bitwise
    step()
    ref = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], k, cfg.score,
                    cfg.renorm, bias=bias, variant=args.variant)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), \
        "staged step differs from moe_forward"
    del ref

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    names = ["route", "permute", "gate_up", "down", "combine"]
    stage_ms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)]))
                for j, n in enumerate(names)}
    ms_step = wall * 1000.0 / K
    value = T / (ms_step / 1000.0)

    # The same step with the load-dependent variant of both expert GEMMs
    # (experts with at most 32 tokens split along K by their token count, the
    # parts added in a second pass): the throughput invariance costs, and how
    # many output elements and probe bits move.  Timed with the same events
    # per step as the invariant step.
    variant_res = None
    if args.variant == 0 and not args.step_only:
        out_inv = out.clone()
        ws_sv = M.workspace(M.OP_GROUPED_SWIGLU, T, H, E, F, k, 1)

        def step_variant(ev=None):
            if ev is not None:
                ev[0].record(stream)
            M.route(x, L["w_router"], k, cfg.score, cfg.renorm, bias=bias, topk_ids=ids,
                    topk_w=w, ws=ws_r)
            if ev is not None:
                ev[1].record(stream)
            M.permute(ids, E, counts, offsets, perm, inv, ws=ws_p)
            if ev is not None:
                ev[2].record(stream)
            M.grouped_swiglu(x, perm, offsets, L["w_gate"], L["w_up"], L["w_down"], k,
                             variant=1, y=y, ws=ws_sv)
            if ev is not None:
                ev[3].record(stream)
                ev[4].record(stream)
            M.combine(y, w, out=out)
            if ev is not None:
                ev[5].record(stream)

        step_variant()
        ref_v = M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], k, cfg.score,
                          cfg.renorm, bias=bias, variant=1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_v.view(torch.int16)), \
            "staged variant step differs from moe_forward"
        del ref_v
        for _ in range(2):
            step_variant()
        KV = min(K, 10)
        evv = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(KV)]
        torch.cuda.synchronize()
        tv = time.perf_counter()
        for i in range(KV):
            step_variant(evv[i])
        torch.cuda.synchronize()
        ms_var = (time.perf_counter() - tv) * 1000.0 / KV
        gemm_var = float(np.mean([evv[i][2].elapsed_time(evv[i][3]) for i in range(KV)]))
        moved = int((out.view(torch.int16) != out_inv.view(torch.int16)).sum().item())
        vbits = None
        if not args.no_check:
            vb = out.view(torch.int16).cpu().numpy()
            vbits = 0
            for i in range(n_probe):
                o1 = M.forward(probes[i:i + 1].contiguous(), L["w_router"], L["w_gate"],
                               L["w_up"], L["w_down"], k, cfg.score, cfg.renorm, bias=bias,
                               variant=1)
                a1 = o1.view(torch.int16).cpu().numpy()[0]
                vbits += int(np.unpackbits(np.bitwise_xor(a1, vb[probe_pos[i]]).view(np.uint8)).sum())
        variant_res = {"kind": "load-dependent split-K of both GEMMs for experts <= 32 tokens",
                       "ms_per_step": round(ms_var, 4), "gemms_ms": round(gemm_var, 4),
                       "invariant_over_variant_throughput": round(ms_var / ms_step, 4),
                       "invariant_over_variant_gemms": round(
                           gemm_var / (stage_ms["gate_up"] + stage_ms["down"]), 4),
                       "out_elements_differing": moved, "out_elements": T * H,
                       "probe_bits_differing": vbits}
        out.copy_(out_inv)

    # Router replay: the same layer with the recorded routing of the step (ids
    # and weights) handed back in; must reproduce the routed output bitwise.
    replay_res = None
    if args.variant == 0 and not args.step_only:
        ws_f = M.workspace(M.OP_FORWARD, T, H, E, F, k)
        rep = M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"], topk_w=w,
                               score=cfg.score, renormalize=cfg.renorm, ws=ws_f)
        same = bool(torch.equal(rep.view(torch.int16), out.view(torch.int16)))
        KR = min(K, 10)
        torch.cuda.synchronize()
        tr = time.perf_counter()
        for _ in range(KR):
            M.forward_replay(x, ids, L["w_gate"], L["w_up"], L["w_down"], topk_w=w,
                             score=cfg.score, renormalize=cfg.renorm, ws=ws_f)
        torch.cuda.synchronize()
        replay_res = {"ms_per_step": round((time.perf_counter() - tr) * 1000.0 / KR, 4),
                      "out_bit_identical_to_routed": same}
        del ws_f, rep

    # The same step as one captured HIP graph (moe_forward on the launch
    # stream, workspace and output preallocated), replayed: the launches'
    # gaps are what it removes, so it matters at decode sizes.  Every replay
    # must give the step's output bit for bit.
    graph_res = None
    if args.variant == 0 and not args.step_only:
        ws_g = M.workspace(M.OP_FORWARD, T, H, E, F, k)
        out_g = torch.empty_like(out)
        fwd = lambda: M.forward(x, L["w_router"], L["w_gate"], L["w_up"], L["w_down"], k,
                                cfg.score, cfg.renorm, bias=bias, out=out_g, ws=ws_g)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fwd()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd()
        out_g.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        same_g = bool(torch.equal(out_g.view(torch.int16), out.view(torch.int16)))
        KG = K
        gs = torch.cuda.current_stream()
        eg = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        eg[0].record(gs)
        for _ in range(KG):
            graph.replay()
        eg[1].record(gs)
        torch.cuda.synchronize()
        g_ms = eg[0].elapsed_time(eg[1]) / KG
        graph_res = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(T / (g_ms * 1e-3), 1),
                     "staged_over_graph_ms": round(ms_step / g_ms, 4),
                     "out_bit_identical": same_g}
        del graph, ws_g, out_g

    # Sparse-indexer top-k at the pages' shape (top 2048 per query over a
    # 128K-token context; 1024 queries), timed on its own.
    topk_res = None
    if cfg.name == "large" and not args.step_only:
        Qs, Ns, ks = 1024, 131072, 2048
        sc = torch.randn((Qs, Ns), generator=torch.Generator().manual_seed(3)).to(dev)
        M.topk_large(sc, ks, want_vals=False)
        evk = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        evk[0].record(stream)
        for _ in range(5):
            M.topk_large(sc, ks, want_vals=False)
        evk[1].record(stream)
        torch.cuda.synchronize()
        tk_ms = evk[0].elapsed_time(evk[1]) / 5
        topk_res = {"queries": Qs, "keys": Ns, "k": ks, "ms": round(tk_ms, 4),
                    "scores_read_once_hbm_frac": round(Qs * Ns * 4.0 / (tk_ms * 1e-3) / 1e9
                                                       / PEAK_HBM_GBS, 4)}
        del sc

    # FP8 rollout path: the same step with e4m3 experts (weights quantised
    # once, at load time, in 128 x 128 blocks; x and act by rows), staged as
    # the entry points moe_forward_fp8 chains and checked bitwise against it;
    # its output against the bf16 layer's, and probe invariance.
    fp8_res, out8 = None, None
    if args.variant == 0 and cfg.name in ("large", "dec") and not args.step_only:
        tq = time.perf_counter()
        wq8 = M.quantize_weights_fp8(L["w_gate"], L["w_up"], L["w_down"])
        torch.cuda.synchronize()
        wq_s = time.perf_counter() - tq
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xe = torch.empty((T, H // 128), dtype=torch.int8, device=dev)
        aq = torch.empty((A, F), dtype=torch.uint8, device=dev)
        ae = torch.empty((A, F // 128), dtype=torch.int8, device=dev)
        out8 = torch.empty_like(out)
        ws_g8 = M.workspace(M.OP_GATE_UP_FP8, T, H, E, F, k)
        ws_d8 = M.workspace(M.OP_DOWN_FP8, T, H, E, F, k)

        def step8(ev=None):
            if ev is not None:
                ev[0].record(stream)
            M.route(x, L["w_router"], k, cfg.score, cfg.renorm, bias=bias, topk_ids=ids,
                    topk_w=w, ws=ws_r)
            if ev is not None:
                ev[1].record(stream)
            M.quantize_fp8(x, 1, q=xq, e=xe)
            if ev is not None:
                ev[2].record(stream)
            M.permute(ids, E, counts, offsets, perm, inv, ws=ws_p)
            if ev is not None:
                ev[3].record(stream)
            M.expert_gate_up_fp8(xq, xe, perm, offsets, wq8["wg_q"], wq8["wg_e"], wq8["wu_q"],
                                 wq8["wu_e"], k, act_q=aq, act_e=ae, ws=ws_g8)
            if ev is not None:
                ev[4].record(stream)
            M.expert_down_fp8(aq, ae, perm, offsets, wq8["wd_q"], wq8["wd_e"], k, y=y,
                              ws=ws_d8)
            if ev is not None:
                ev[5].record(stream)
            M.combine(y, w, out=out8)
            if ev is not None:
                ev[6].record(stream)

        step8()
        ref8 = M.forward_fp8(x, L["w_router"], wq8, k, cfg.score, cfg.renorm, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(out8.view(torch.int16), ref8.view(torch.int16)), \
            "staged FP8 step differs from moe_forward_fp8"
        del ref8
        for _ in range(2):
            step8()
        K8 = max(3, min(K, 10))
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(K8)]
        torch.cuda.synchronize()
        t8 = time.perf_counter()
        for i in range(K8):
            step8(ev8[i])
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t8) * 1000.0 / K8
        n8 = ["route", "quantize_x", "permute", "gate_up_fp8", "down_fp8", "combine"]
        st8 = {n: float(np.mean([ev8[i][j].elapsed_time(ev8[i][j + 1]) for i in range(K8)]))
               for j, n in enumerate(n8)}
        gu8 = 4.0 * A * H * F / (st8["gate_up_fp8"] * 1e-3) / 1e12
        dn8 = 2.0 * A * H * F / (st8["down_fp8"] * 1e-3) / 1e12
        o8, o16 = out8.float(), out.float()
        rel = float((o8 - o16).norm() / o16.norm())
        nd8 = 0
        b8 = out8.view(torch.int16).cpu().numpy()
        for i in range(min(4, n_probe)):
            p1 = M.forward_fp8(probes[i:i + 1].contiguous(), L["w_router"], wq8, k, cfg.score,
                               cfg.renorm, bias=bias)
            a1 = p1.view(torch.int16).cpu().numpy()[0]
            b1 = b8[probe_pos[i]]
            nd8 += int(np.unpackbits(np.bitwise_xor(a1, b1).view(np.uint8)).sum())
        fp8_res = {"ms_per_step": round(ms8, 4), "tokens_per_s": round(T / (ms8 * 1e-3), 1),
                   "stages_ms": {n: round(v, 4) for n, v in st8.items()},
                   "gate_up_fp8_tflops": round(gu8, 2),
                   "gate_up_fp8_mfma_frac": round(gu8 / PEAK_FP8_TFLOPS, 4),
                   "down_fp8_tflops": round(dn8, 2),
                   "down_fp8_mfma_frac": round(dn8 / PEAK_FP8_TFLOPS, 4),
                   "speedup_vs_bf16_step": round(ms_step / ms8, 3),
                   "out_rel_diff_vs_bf16": round(rel, 5),
                   "probe_bits_differing": nd8,
                   "weight_quantise_s": round(wq_s, 3)}
        del wq8, xq, xe, aq, ae, ws_g8, ws_d8

    # Decode workload: the measurement downstream of the step (vocabulary
    # projection, log-softmax, k3 of this batch against itself), timed on its
    # own; the projection streams V x H bf16 weights.
    decode_res = None
    if cfg.name == "dec" and not args.step_only:
        V = 65536
        gp = torch.Generator().manual_seed(I.PROJ_SEED)
        P = torch.randn((V, H), generator=gp).to(torch.bfloat16).to(dev)
        z = torch.empty((T, V), dtype=torch.float32, device=dev)
        lp = torch.empty_like(z)
        ws_ls = M.workspace(M.OP_LOG_SOFTMAX, T, V, 1, 64, 1)
        ws_k3 = M.workspace(M.OP_K3, T, V, 1, 64, 1)
        for _ in range(2):
            M.lm_head_logits(out, P, z=z)
            M.log_softmax(z, out=lp, ws=ws_ls)
            M.k3(lp, lp, ws=ws_k3)
        KD = max(5, min(K, 20))
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(KD)]
        torch.cuda.synchronize()
        for i in range(KD):
            evd[i][0].record(stream)
            M.lm_head_logits(out, P, z=z)
            evd[i][1].record(stream)
            M.log_softmax(z, out=lp, ws=ws_ls)
            evd[i][2].record(stream)
            kmean, _, _ = M.k3(lp, lp, ws=ws_k3)
            evd[i][3].record(stream)
        torch.cuda.synchronize()
        dms = [float(np.mean([evd[i][j].elapsed_time(evd[i][j + 1]) for i in range(KD)]))
               for j in range(3)]
        proj_bytes = 2.0 * V * H
        if out8 is not None:
            # the gap the FP8 rollout leaves against the BF16 policy: k3 of the
            # FP8 layer's next-token distribution against the BF16 layer's
            lp8 = M.log_softmax(M.lm_head_logits(out8, P))
            k3m, _, g8 = M.k3(lp, lp8)
            _, _, g16 = M.k3(lp, lp)
            fp8_res["decode_k3_vs_bf16"] = {
                "k3_mean": float(k3m.mean().item()), "k3_max": float(k3m.max().item()),
                "greedy_agree": float((g8 == g16).float().mean().item())}
            del lp8
        decode_res = {"vocab": V, "lm_head_ms": round(dms[0], 4),
                      "lm_head_hbm_frac": round(proj_bytes / (dms[0] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "lm_head_kernel": ("valu fma, one row per thread" if 4 < T <= 8 else
                                         "valu fma, whole-line loads through LDS"
                                         if T <= 4 or (T <= 16 and V >= 16384)
                                         else "mfma_f32 32x32x1"),
                      "lm_head_fp32_tflops": round(2.0 * T * V * H / (dms[0] * 1e-3) / 1e12, 2),
                      "log_softmax_ms": round(dms[1], 4),
                      "log_softmax_hbm_frac": round(8.0 * T * V / (dms[1] * 1e-3) / 1e9
                                                    / PEAK_HBM_GBS, 4),
                      "k3_ms": round(dms[2], 4),
                      "k3_self": float(kmean.max().item())}
        del P, z, lp

    counts_np = counts.cpu().numpy()
    gu_flops = 4.0 * A * H * F
    dn_flops = 2.0 * A * H * F
    gu_tflops = gu_flops / (stage_ms["gate_up"] * 1e-3) / 1e12
    grouped_tflops = (gu_flops + dn_flops) / ((stage_ms["gate_up"] + stage_ms["down"]) * 1e-3) / 1e12
    comb_bytes = 4.0 * A * H + 4.0 * A + 2.0 * T * H
    comb_gbs = comb_bytes / (stage_ms["combine"] * 1e-3) / 1e9
    # permute: ids read, perm and inv_perm written (4 B each per assignment),
    # counts and offsets (8 B per expert)
    perm_bytes = 12.0 * A + 8.0 * E
    perm_gbs = perm_bytes / (stage_ms["permute"] * 1e-3) / 1e9

    # The gate/up kernel's bound is the larger of its two floors: the MFMA time
    # of its flops and the HBM time of its algorithmic bytes (the active
    # experts' gate and up weights + x + h_act).  MFMA at prefill sizes; at
    # decode sizes it streams the weights.
    active = int((counts_np > 0).sum())
    gu_bytes = active * 2.0 * F * H * 2 + 2.0 * T * H + 2.0 * A * F
    t_mfma = gu_flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = gu_bytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_mfma:
        gu_gbs = gu_bytes / (stage_ms["gate_up"] * 1e-3) / 1e9
        roofline = {"kernel": "expert_gemm_pipe_kernel<0> (moe_expert_gate_up)",
                    "bound": "hbm", "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gu_gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic_bytes(cfg.name, T)}
    else:
        roofline = {"kernel": "expert_gemm_pipe_kernel<0> (moe_expert_gate_up)",
                    "bound": "mfma", "achieved": round(gu_tflops, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_bytes(cfg.name, T)}

    # batch invariance of the embedded probes: each probe alone (T = 1) vs in the batch
    inv_bits = None
    if not args.no_check and args.variant == 0:
        batch_bits = out.view(torch.int16).cpu().numpy()
        nd = 0
        for i in range(n_probe):
            o1 = M.forward(probes[i:i + 1].contiguous(), L["w_router"], L["w_gate"], L["w_up"],
                           L["w_down"], k, cfg.score, cfg.renorm, bias=bias)
            a = o1.view(torch.int16).cpu().numpy()[0]
            b = batch_bits[probe_pos[i]]
            nd += int(np.unpackbits(np.bitwise_xor(a, b).view(np.uint8)).sum())
        inv_bits = nd

    # router logits: fp32 fma chains in the pinned order, on the matrix cores
    # (K=1 fp32 MFMA, the same chains bit for bit) where the library's route
    # plan takes them, else on the VALU (packed fp32 is not used); and the
    # bytes of x and w_router
    r_flops = 2.0 * T * H * E
    r_bytes = 2.0 * T * H + 2.0 * E * H
    r_s = stage_ms["route"] * 1e-3
    mfma_route = route_uses_matrix_cores(T, H, E)
    r_peak = PEAK_FP32_MFMA_TFLOPS if mfma_route else PEAK_FP32_VALU_TFLOPS
    route_res = {"kernel": "mfma_f32 32x32x1" if mfma_route else "valu fma",
                 "fp32_tflops": round(r_flops / r_s / 1e12, 2),
                 "frac": round(r_flops / r_s / 1e12 / r_peak, 4),
                 "peak_tflops": r_peak,
                 "valu_frac": round(r_flops / r_s / 1e12 / PEAK_FP32_VALU_TFLOPS, 4),
                 "hbm_frac": round(r_bytes / r_s / 1e9 / PEAK_HBM_GBS, 4),
                 "binds": ("mfma_f32" if mfma_route else "valu")
                          if r_flops / (r_peak * 1e12) > r_bytes / (PEAK_HBM_GBS * 1e9) else "hbm"}

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} H={H} E={E} top-{k} F={F} "
                               f"{'sigmoid+Zipf(1.2) bias' if cfg.score else 'softmax'}"
                               f"{' renorm' if cfg.renorm else ''}",
                   "variant": "invariant" if args.variant == 0 else "load-dependent",
                   "active_experts": int((counts_np > 0).sum()),
                   "max_expert_tokens": int(counts_np.max())},
        # the realised routing load: experts per token-count bucket, and the largest loads
        "expert_load": {
            "experts_by_tokens": {
                label: int(((counts_np >= lo) & (counts_np < hi)).sum())
                for label, lo, hi in (("0", 0, 1), ("1-63", 1, 64), ("64-255", 64, 256),
                                      ("256-1023", 256, 1024), ("1024-4095", 1024, 4096),
                                      (">=4096", 4096, 1 << 31))},
            "largest": [int(v) for v in np.sort(counts_np)[::-1][:8]]},
        "roofline": roofline,
        "stages_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "route": route_res,
        "grouped_gemm_tflops": round(grouped_tflops, 2),
        "grouped_gemm_mfma_frac": round(grouped_tflops / PEAK_BF16_TFLOPS, 4),
        "combine_hbm_frac": round(comb_gbs / PEAK_HBM_GBS, 4),
        "permute_hbm_frac": round(perm_gbs / PEAK_HBM_GBS, 5),
        "gemm_source_hash": gemm_source_hash()[:16],
        "probe_bits_differing": inv_bits,
        "variant": variant_res,
        "router_replay": replay_res,
        "graph_replay": graph_res,
        "indexer_topk": topk_res,
        "fp8_experts": fp8_res,
    }
    if decode_res is not None:
        res["decode_measure"] = decode_res

    # oracle on the host cores, bounded sample of the same workload: timed at
    # every host thread and at one, and compared with the GPU's rows (parity
    # of the timed step's own output)
    nsample = args.cpu_sample
    if nsample is None:
        # about 10-15 s of oracle work on 16 host threads (the large layer's
        # whole-layer oracle runs ~27 tokens/s there; the tie and mid layers
        # cost 0.66x and 0.23x as much per token); at most the batch
        nsample = {"large": 320, "dec": 64, "tie": 480, "mid": 1400, "tiny": 64}[cfg.name]
    nsample = min(nsample, T)
    if nsample > 0:
        from oracle import oracle as O
        xb = I.bf16_bits(x)
        hb = {n: I.bf16_bits(t) for n, t in L.items() if t is not None and t.dtype == torch.bfloat16}
        bias_np = bias.cpu().numpy() if bias is not None else None
        rows = np.sort(np.random.default_rng(0).choice(T, nsample, replace=False))
        nthreads = O.max_threads()
        c0 = time.perf_counter()
        out_r, ids_r, w_r, gap = O.forward_tokens(rows, xb, hb["w_router"], hb["w_gate"],
                                                  hb["w_up"], hb["w_down"], k, cfg.score,
                                                  cfg.renorm, bias=bias_np, nthreads=nthreads)
        cdt = time.perf_counter() - c0
        # one thread, on the first rows of the same sample (about half the time)
        n1 = max(1, min(nsample, int(round(nsample / cdt * 0.5 / max(nthreads, 1)))))
        c1 = time.perf_counter()
        O.forward_tokens(rows[:n1], xb, hb["w_router"], hb["w_gate"], hb["w_up"], hb["w_down"],
                         k, cfg.score, cfg.renorm, bias=bias_np, nthreads=1)
        cdt1 = time.perf_counter() - c1
        res["cpu_baseline"] = {"value": round(nsample / cdt, 3), "unit": "tokens/s",
                               "cores": nthreads, "kind": "oracle",
                               "sample": f"{nsample} of the {T} tokens, whole layer per token "
                                         f"(route over all {E} experts, {k} expert FFNs, "
                                         f"combine), {cdt:.1f}s on {nthreads} threads",
                               "one_thread": {"value": round(n1 / cdt1, 3), "tokens": n1,
                                              "s": round(cdt1, 2)},
                               "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}
        # parity of the sample: ids bit-exact except near-tie exemptions (gap
        # below 1e-6; the tie layer's constructed stress tokens are never
        # exempt), out within 2e-2 + 1e-2 |ref| per element
        g_ids = ids.cpu().numpy()[rows]
        g_out = I.bf16_bits(out)[rows]
        exempt = gap < 1e-6
        if cfg.name == "tie":
            exempt &= d["kind"][rows] < 2
        mism = np.any(g_ids != ids_r, axis=1)
        same = ~mism
        go = O.bf16_to_f32(g_out[same]).astype(np.float64)
        ro = O.bf16_to_f32(out_r[same]).astype(np.float64)
        err = np.abs(go - ro)
        gw = w.cpu().numpy()[rows][same].astype(np.float64)
        rw = w_r[same].astype(np.float64)
        res["parity"] = {
            "rows": int(nsample), "id_mismatches": int((mism & ~exempt).sum()),
            "exempt_tokens": int(exempt.sum()), "exempt_mismatches": int((mism & exempt).sum()),
            "max_abs_err": float(err.max()) if err.size else 0.0,
            "max_rel_err": float((err / np.maximum(np.abs(ro), 1e-30))[np.abs(ro) > 0].max())
            if err.size else 0.0,
            "out_of_tolerance": int((err > 2e-2 + 1e-2 * np.abs(ro)).sum()),
            "out_bit_identical": round(float(np.mean(g_out[same] == out_r[same])), 5),
            "weights_max_rel_err": float((np.abs(gw - rw) / np.maximum(np.abs(rw), 1e-30)).max())
            if rw.size else 0.0}
        if cfg.name == "tie":
            st = d["kind"][rows] >= 2
            res["parity"]["stress_tokens"] = int(st.sum())
            res["parity"]["stress_id_mismatches"] = int((mism & st).sum())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
