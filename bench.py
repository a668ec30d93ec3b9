#!/usr/bin/env python3
"""Benchmark of the MoonEP balanced expert-parallel hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic routing:
plan -> weight prefetch -> dispatch -> grouped SwiGLU GEMM -> combine, then the
backward: scaled dispatch of dOut -> grouped GEMM backward (dX, dW) -> unit combine
-> reduce_grad.  Workload: R=8 emulated EP ranks, E=256 experts, B=4 slots, S=4096
tokens/rank, K=8, H=7168, I=2048, bf16, router bias tuned to expert-level maxvio 4.

Prints ONE JSON line.  value = dispatch+combine GB/s (algorithmic bytes of all four
permute/unpermute calls of a step over their HIP-event time); also the grouped GEMM
TFLOP/s, a maxvio sweep, per-call rooflines, and the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--maxvio", type=float, default=4.0)
    p.add_argument("--no-sweep", action="store_true", help="skip the maxvio sweep")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-tokens", type=int, default=512, help="tokens per rank in the CPU sample")
    return p.parse_args()


class Timer:
    """HIP events on torch's current stream (the stream every library call is launched on)."""

    def __init__(self, torch):
        self.torch = torch
        self.rec = {}

    def run(self, name, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.rec.setdefault(name, []).append((a, b))

    def clear(self):
        self.rec = {}

    def avg_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.rec.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the R expert-parallel ranks are emulated as "
              f"partitions of a single MI355X, so --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import balanced_token_dispatch_moonep_amd as M
    from balanced_token_dispatch_moonep_amd.layer import MoonEPLayer
    import workload as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS["train"].with_(maxvio=args.maxvio)
    R, E, B, S, K, H, I = cfg.R, cfg.E, cfg.B, cfg.S, cfg.K, cfg.H, cfg.I
    Mrows = R * S * K

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    log(f"[bench] workload R{R} E{E} B{B} S{S} K{K} H{H} I{I} maxvio {args.maxvio}")
    topk, gates, lam = W.routing_for(cfg)
    xb = W.hidden_rows(R, S, H, cfg.seed, "bf16")
    db = W.grad_rows(R, S, H, cfg.seed, "bf16")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x, dout = bf(xb), bf(db)
    tk = torch.from_numpy(topk).to(dev)
    g = torch.from_numpy(gates).to(dev)
    w13, w2 = W.expert_weights_torch(E, H, I, cfg.seed, dev)
    d = M.Dims.make(R, E, B, S, K, H, I, training=True)
    L = MoonEPLayer(d, w13=w13, w2=w2, training=True)
    log("[bench] inputs resident; warming up")

    T = Timer(torch)

    def step():
        T.run("plan", lambda: L.plan(tk))
        T.run("prefetch", L.prefetch)
        T.run("dispatch", lambda: L.dispatch(x))
        T.run("ffn_fwd", L.expert_ffn)
        T.run("combine", lambda: L.combine(g))
        T.run("dispatch_bwd", lambda: M.moonep_dispatch(d, L.dest, dout, g, L.dy))
        T.run("ffn_bwd", lambda: M.moonep_grouped_ffn_backward(
            d, L.ws, L.cu, L.recv, L.gu, L.act, L.dy, L.w13, L.w2, L.w13_slot, L.w2_slot, L.drecv,
            L.dw13, L.dw2, L.dw13_red, L.dw2_red))
        T.run("combine_bwd", lambda: M.moonep_combine(d, L.dest, L.drecv, None, L.dx))
        T.run("reduce_grad", lambda: M.moonep_reduce_grad(d, L.ws, L.dw13, L.dw2, L.dw13_red, L.dw2_red))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = L.stats.cpu().numpy()
    T.clear()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = T.avg_ms()
    ms_step = wall * 1e3 / args.steps
    log("[bench] per-call ms:", {k: round(v, 4) for k, v in ms.items()}, "step ms", round(ms_step, 3))

    # algorithmic work per call (what the method must move or compute)
    xbytes = R * S * H * 2
    rbytes = Mrows * H * 2
    NW = 3 * H * I
    n_slot = int(st[2])
    work = {
        "plan": ("hbm", 8.0 * Mrows),
        "prefetch": ("hbm", 2.0 * n_slot * NW * 2),
        "dispatch": ("hbm", xbytes + rbytes + 4.0 * Mrows),
        "combine": ("hbm", rbytes + 8.0 * Mrows + xbytes),
        "dispatch_bwd": ("hbm", xbytes + rbytes + 8.0 * Mrows),
        "combine_bwd": ("hbm", rbytes + 4.0 * Mrows + xbytes),
        "ffn_fwd": ("mfma", 6.0 * Mrows * H * I),
        "ffn_bwd": ("mfma", 12.0 * Mrows * H * I),
    }
    # reduce_grad: (8 + 8n) * NW bytes for every expert with n slot replicas; the slot
    # replicas per expert are read off the device plan (slot rows of cu_seqlens, and the
    # expert of their first row via dest).
    cu = L.cu.cpu().numpy()
    dst = L.dest.cpu().numpy().ravel()
    tkf = topk.ravel()
    row_expert = np.full(Mrows, -1, dtype=np.int64)
    row_expert[dst] = tkf
    reps = {}
    for q in range(R):
        for j in range(B):
            lo, hi = cu[q, E + j], cu[q, E + j + 1]
            if hi > lo:
                e = int(row_expert[q * S * K + lo])
                reps[e] = reps.get(e, 0) + 1
    work["reduce_grad"] = ("hbm", float(sum((8 + 8 * n) * NW for n in reps.values())))

    rooflines = {}
    for k, (bound, amount) in work.items():
        t = ms.get(k, 0.0) / 1e3
        if bound == "hbm":
            ach = amount / t / 1e9 if t > 0 else 0.0
            rooflines[k] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(ach / HBM_PEAK_GBS, 4), "ms": round(ms[k], 4), "bytes": amount}
        else:
            ach = amount / t / 1e12 if t > 0 else 0.0
            rooflines[k] = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                            "ms": round(ms[k], 4), "flops": amount}
    dc_keys = ("dispatch", "combine", "dispatch_bwd", "combine_bwd")
    dc_bytes = sum(work[k][1] for k in dc_keys)
    dc_ms = sum(ms[k] for k in dc_keys)
    value = dc_bytes / (dc_ms / 1e3) / 1e9
    gemm_tflops = (work["ffn_fwd"][1] + work["ffn_bwd"][1]) / ((ms["ffn_fwd"] + ms["ffn_bwd"]) / 1e3) / 1e12
    dom = max(ms, key=lambda k: ms[k])
    r = rooflines[dom]
    roofline = {"bound": r["bound"], "achieved": r["achieved"], "peak": r["peak"], "unit": r["unit"],
                "frac": r["frac"], "traffic": None, "kernel": f"moonep_{dom}" if not dom.endswith("_bwd")
                else "moonep_grouped_ffn_backward" if dom == "ffn_bwd" else f"moonep_{dom}"}

    # ---- maxvio sweep (same shapes): plan, dispatch+combine, GEMM forward -------------------
    sweep = []
    if not args.no_sweep:
        for mv in (0.0, 0.5, 2.0, 4.0, 8.0):
            c2 = cfg.with_(maxvio=mv)
            tk2, g2, lam2 = W.routing_for(c2)
            tkd, gd = torch.from_numpy(tk2).to(dev), torch.from_numpy(g2).to(dev)
            T2 = Timer(torch)
            for it in range(4):
                T2.run("plan", lambda: L.plan(tkd))
                T2.run("prefetch", L.prefetch)
                T2.run("dispatch", lambda: L.dispatch(x))
                T2.run("ffn_fwd", L.expert_ffn)
                T2.run("combine", lambda: L.combine(gd))
                if it == 0:
                    torch.cuda.synchronize()
                    T2.clear()
            torch.cuda.synchronize()
            m2 = T2.avg_ms()
            s2 = L.stats.cpu().numpy()
            Lx = np.bincount(tk2.ravel(), minlength=E).astype(np.float64)
            sweep.append({
                "maxvio": round(float((Lx.max() - Lx.mean()) / Lx.mean()), 3), "lambda": round(lam2, 4),
                "replicas": int(s2[1]), "fallback_replicas": int(s2[3]),
                "migrated_frac": round(int(s2[5]) / Mrows, 4),
                "rank_peak_over_mean": round(int(s2[8]) / (S * K), 4),
                "plan_us": round(m2["plan"] * 1e3, 1), "prefetch_ms": round(m2["prefetch"], 4),
                "dispatch_ms": round(m2["dispatch"], 4), "combine_ms": round(m2["combine"], 4),
                "dc_GBps": round((work["dispatch"][1] + work["combine"][1]) /
                                 ((m2["dispatch"] + m2["combine"]) / 1e3) / 1e9, 1),
                "gemm_fwd_ms": round(m2["ffn_fwd"], 3),
                "gemm_fwd_TFLOPs": round(work["ffn_fwd"][1] / (m2["ffn_fwd"] / 1e3) / 1e12, 1),
            })
            log("[bench] sweep", sweep[-1])

    # ---- CPU oracle baseline on a bounded sample of the same workload ----------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, args.cpu_tokens, log)

    out = {
        "metric": "dispatch+combine GB/s and grouped-GEMM TFLOP/s vs maxvio, % of roofline, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded router logits N(0,1) + Zipf expert bias, bf16 N(0,1) rows, N(0,0.02) weights)",
        "config": {"workload": "moe_layer_train_fwd_bwd", "R": R, "E": E, "B": B, "S": S, "K": K, "H": H,
                   "I": I, "maxvio": round(float(np.bincount(topk.ravel(), minlength=E).max() /
                                                 (R * S * K / E) - 1), 3),
                   "replicas": int(st[1]), "fallback_replicas": int(st[3]), "parallelism": "ep8-emulated-1gpu"},
        "dc_GBps": round(value, 1),
        "dc_frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_mfma": round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roofline,
        "rooflines": rooflines,
        "sweep": sweep,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(cfg, tokens, log):
    """The CPU oracle, as it stands, on the same workload with `tokens` tokens per rank."""
    import numpy as np
    import oracle as O
    import workload as W
    c = cfg.with_(S=tokens)
    R, E, B, S, K, H, I = c.R, c.E, c.B, c.S, c.K, c.H, c.I
    topk, gates, _ = W.routing_for(c)
    xb = W.hidden_rows(R, S, H, c.seed, "bf16")
    t0 = time.perf_counter()
    plan = O.make_plan(topk, E, B, training=True)
    dest = O.destinations(topk, plan)
    t1 = time.perf_counter()
    recv = O.dispatch(dest, xb)
    t2 = time.perf_counter()
    out = O.combine(dest, recv, gates)
    t3 = time.perf_counter()
    Mr = R * S * K
    dc_bytes = (R * S * H * 2 + Mr * H * 2 + 4 * Mr) + (Mr * H * 2 + 8 * Mr + R * S * H * 2)
    # expert FFN forward on the first few groups (weights drawn for those experts only)
    grp = O.groups(plan)[:4]
    rng = np.random.Generator(np.random.PCG64([c.seed, 99]))
    flops = 0.0
    t4 = time.perf_counter()
    for (q, w, row0, rows, kind, idx) in grp:
        w13 = rng.standard_normal((1, H, 2 * I), dtype=np.float32) * np.float32(0.02)
        w2 = rng.standard_normal((1, I, H), dtype=np.float32) * np.float32(0.02)
        sub = O.layer._f64(recv[row0:row0 + rows])
        gq = sub @ w13[0].astype(np.float64)
        a = O.silu(gq[:, :I]) * gq[:, I:]
        _ = a @ w2[0].astype(np.float64)
        flops += 6.0 * rows * H * I
    t5 = time.perf_counter()
    del out
    cores = len(os.sched_getaffinity(0))
    res = {
        "value": round(dc_bytes / (t3 - t1) / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"same workload with S={S} tokens/rank (R{R} E{E} K{K} H{H} maxvio {cfg.maxvio}): "
                  f"plan+destinations, dispatch and combine (value = their bytes / dispatch+combine time); "
                  f"FFN forward on {len(grp)} groups in float64",
        "plan_s": round(t1 - t0, 3),
        "dispatch_s": round(t2 - t1, 3),
        "combine_s": round(t3 - t2, 3),
        "ffn_TFLOPs": round(flops / (t5 - t4) / 1e12, 4),
        "threads": os.environ.get("OMP_NUM_THREADS", str(cores)),
        "cpu_model": platform.processor() or _cpu_model(),
    }
    log("[bench] cpu baseline", res)
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
