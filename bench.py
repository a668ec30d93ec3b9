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
import gc
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


SWEEP = (0.0, 0.5, 2.0, 4.0, 8.0)

# timed call -> the one kernel it launches (name as in rocprofv3 kernel traces); the plan call
# launches three small kernels and has no entry.  The weight-gradient calls also launch a
# one-workgroup kernel that resets their eight per-XCD tile counters and orders their targets
# before the GEMM, the row GEMM calls a one-wave counter reset and a one-wave tile prefix.
KERNEL_NAMES = {
    "prefetch": "moonep::prefetch_kernel",
    "dispatch": "moonep::dispatch_kernel<false, false, 0, 2, false, true>",
    "gemm_gate_up": "moonep::gemm_rows_kernel<0, 0, 4>",
    "gemm_down": "moonep::gemm_rows_kernel<0, 1, 4>",
    "combine": "moonep::combine_kernel<false, true, 7, false, true>",
    "dispatch_bwd": "moonep::dispatch_kernel<false, true, 8, 2, false, true>",
    "gemm_dact": "moonep::gemm_rows_kernel<1, 2, 4>",
    "gemm_dx": "moonep::gemm_rows_kernel<1, 1, 4>",
    "gemm_dw2": "moonep::gemm_dw_kernel<256, 2>",
    "gemm_dw13": "moonep::gemm_dw_kernel<256, 13>",
    "combine_bwd": "moonep::combine_kernel<false, false, 7, false, false>",
    "reduce_grad": "moonep::reduce_grad_kernel",
}
# sources each kernel is compiled from (a code change to any of them, comments aside, voids its
# stored counters)
KERNEL_SOURCES = {
    "prefetch": ("weights.hip",), "reduce_grad": ("weights.hip",),
    "dispatch": ("permute.hip",), "combine": ("permute.hip",),
    "dispatch_bwd": ("permute.hip",), "combine_bwd": ("permute.hip",),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_busy.json")
SIMDS = 256 * 4      # MI355X: 256 compute units of 4 SIMDs
XCDS = 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--maxvio", type=float, default=4.0)
    p.add_argument("--no-sweep", action="store_true", help="skip the maxvio sweep")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-tokens", type=int, default=4096, help="tokens per rank in the CPU sample")
    p.add_argument("--cpu-groups", type=int, default=32, help="expert groups in the CPU FFN sample")
    p.add_argument("--traffic-from", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON"),
                   help="no GPU work: reduce two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then "
                        "WRITE_SIZE) and that run's JSON line to per-launch HBM bytes; writes "
                        "profiles/hbm_traffic.json and prints a markdown summary")
    p.add_argument("--mfma-from", nargs=2, metavar=("PMC_DIR", "BENCH_JSON"),
                   help="no GPU work: reduce a rocprofv3 --pmc run of this bench (SQ_VALU_MFMA_BUSY_CYCLES, "
                        "SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE, with --kernel-trace) and that run's "
                        "JSON line to per-kernel matrix-core busy fractions; writes profiles/mfma_busy.json "
                        "and prints a markdown summary")
    p.add_argument("--stats-from", metavar="DIR",
                   help="no GPU work: print a markdown table of a rocprofv3 --stats kernel summary")
    p.add_argument("--l2-from", nargs=2, metavar=("PMC_DIR1", "PMC_DIR2"),
                   help="no GPU work: reduce two rocprofv3 --pmc runs of this bench (TCC_HIT_sum "
                        "TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum, then TCC_TAG_STALL_sum "
                        "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_LEVEL_sum TCC_EA0_RDREQ_32B_sum, each with "
                        "--kernel-trace) to a markdown table of every GEMM kernel's L2 hit rate, reads "
                        "beyond L2 and their mean latency")
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

    def spread_ms(self):
        """Median and minimum of each call's launches."""
        out = {}
        for k, v in self.rec.items():
            t = sorted(a.elapsed_time(b) for a, b in v)
            n = len(t)
            out[k] = {"median_ms": round((t[(n - 1) // 2] + t[n // 2]) / 2, 4), "min_ms": round(t[0], 4)}
        return out


def main():
    args = parse()
    if args.traffic_from:
        return write_traffic(*args.traffic_from)
    if args.stats_from:
        return print_stats(args.stats_from)
    if args.mfma_from:
        return write_mfma(*args.mfma_from)
    if args.l2_from:
        return print_l2(*args.l2_from)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
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
    bwd_args = lambda: (L.ws, L.cu, L.recv, L.gu, L.act, L.dy, L.w13, L.w2, L.w13_slot, L.w2_slot, L.drecv,
                        L.dw13, L.dw2, L.dw13_red, L.dw2_red)
    dph = {ph: d.with_flags(d.flags | ph) for ph in (M.PHASE_GATE_UP, M.PHASE_DOWN, M.PHASE_DACT, M.PHASE_DX,
                                                   M.PHASE_DW2, M.PHASE_DW13)}

    def ffn_fwd_phase(ph):
        M.moonep_grouped_ffn(dph[ph], L.ws, L.cu, L.recv, L.w13, L.w2, L.w13_slot, L.w2_slot, L.gu, L.act, L.y)

    def ffn_bwd_phase(ph):
        M.moonep_grouped_ffn_backward(dph[ph], *bwd_args())

    def step(T, gates, tkd, backward=True):
        # every GEMM phase is its own call, so each kernel is timed on its own
        T.run("plan", lambda: L.plan(tkd))
        T.run("prefetch", L.prefetch)
        T.run("dispatch", lambda: L.dispatch(x))
        T.run("gemm_gate_up", lambda: ffn_fwd_phase(M.PHASE_GATE_UP))
        T.run("gemm_down", lambda: ffn_fwd_phase(M.PHASE_DOWN))
        T.run("combine", lambda: L.combine(gates))
        if not backward:
            return
        T.run("dispatch_bwd", lambda: M.moonep_dispatch(d, L.dest, dout, gates, L.dy))
        T.run("gemm_dact", lambda: ffn_bwd_phase(M.PHASE_DACT))
        T.run("gemm_dx", lambda: ffn_bwd_phase(M.PHASE_DX))
        T.run("gemm_dw2", lambda: ffn_bwd_phase(M.PHASE_DW2))
        T.run("gemm_dw13", lambda: ffn_bwd_phase(M.PHASE_DW13))
        T.run("combine_bwd", lambda: M.moonep_combine(d, L.dest, L.drecv, None, L.dx))
        T.run("reduce_grad", lambda: M.moonep_reduce_grad(d, L.ws, L.dw13, L.dw2, L.dw13_red, L.dw2_red))

    for _ in range(args.warmup):
        step(T, g, tk)
    torch.cuda.synchronize()
    T.clear()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(T, g, tk)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = T.avg_ms()
    st = L.stats.cpu().numpy()
    ms_step = wall * 1e3 / args.steps
    log("[bench] per-call ms:", {k: round(v, 4) for k, v in ms.items()}, "step ms", round(ms_step, 3))

    work = algorithmic_work(cfg, st, L.cu.cpu().numpy(), L.dest.cpu().numpy().ravel(), topk)
    rooflines = {k: roofline_of(k, work[k], ms[k]) for k in ms}
    for k, sp in T.spread_ms().items():
        rooflines[k].update(sp)
    fwd_keys, bwd_keys = ("gemm_gate_up", "gemm_down"), ("gemm_dact", "gemm_dx", "gemm_dw2", "gemm_dw13")
    dc_keys = ("dispatch", "combine", "dispatch_bwd", "combine_bwd")
    dc_bytes = sum(work[k][1] for k in dc_keys)
    dc_ms = sum(ms[k] for k in dc_keys)
    value = dc_bytes / (dc_ms / 1e3) / 1e9
    gemm_keys = fwd_keys + bwd_keys
    gemm_tflops = sum(work[k][1] for k in gemm_keys) / (sum(ms[k] for k in gemm_keys) / 1e3) / 1e12
    fwd_tflops = sum(work[k][1] for k in fwd_keys) / (sum(ms[k] for k in fwd_keys) / 1e3) / 1e12
    bwd_tflops = sum(work[k][1] for k in bwd_keys) / (sum(ms[k] for k in bwd_keys) / 1e3) / 1e12
    # dominant kernel: the single-kernel call with the longest average launch
    dom = max((k for k in ms if k in KERNEL_NAMES), key=lambda k: ms[k])
    r = rooflines[dom]
    roofline = {"bound": r["bound"], "achieved": r["achieved"], "peak": r["peak"], "unit": r["unit"],
                "frac": r["frac"], "traffic": traffic_of(dom, work[dom][2]), "kernel": KERNEL_NAMES[dom],
                "call": dom, "ms": r["ms"], "per_launch": work[dom][3]}
    if r["bound"] == "mfma":
        roofline["mfma_busy"] = stored_of(MFMA_FILE, dom, "mfma_busy_frac")
    for k in gemm_keys:
        rooflines[k]["mfma_busy"] = stored_of(MFMA_FILE, k, "mfma_busy_frac")

    # ---- maxvio sweep (same shapes): the whole training step per maxvio ----------------------
    sweep = []
    if not args.no_sweep:
        for mv in SWEEP:
            c2 = cfg.with_(maxvio=mv)
            tk2, g2, lam2 = W.routing_for(c2)
            tkd, gd = torch.from_numpy(tk2).to(dev), torch.from_numpy(g2).to(dev)
            T2 = Timer(torch)
            step(T2, gd, tkd)
            torch.cuda.synchronize()
            T2.clear()
            for it in range(3):
                step(T2, gd, tkd)
            torch.cuda.synchronize()
            m2 = T2.avg_ms()
            s2 = L.stats.cpu().numpy()
            cu2 = L.cu.cpu().numpy()
            w2k = algorithmic_work(c2, s2, cu2, L.dest.cpu().numpy().ravel(), tk2)
            sweep.append(sweep_entry(c2, tk2, lam2, s2, m2, w2k, "train", cu2))
            log("[bench] sweep", sweep[-1])
        # inference variant: B = 3 prefetch slots, fallback replicas read their home rows
        ci = cfg.with_(B=3)
        di = M.Dims.make(R, E, 3, S, K, H, I, training=False)
        Li = MoonEPLayer(di, w13=w13, w2=w2, training=False)
        Ti = Timer(torch)
        for it in range(4):
            Ti.run("plan", lambda: Li.plan(tk))
            Ti.run("prefetch", Li.prefetch)
            Ti.run("dispatch", lambda: Li.dispatch(x))
            Ti.run("ffn_fwd", Li.expert_ffn)
            Ti.run("combine", lambda: Li.combine(g))
            if it == 0:
                torch.cuda.synchronize()
                Ti.clear()
        torch.cuda.synchronize()
        si = Li.stats.cpu().numpy()
        cui = Li.cu.cpu().numpy()
        wi = algorithmic_work(ci, si, cui, Li.dest.cpu().numpy().ravel(), topk)
        sweep.append(sweep_entry(ci, topk, lam, si, Ti.avg_ms(), wi, "inference_B3", cui))
        log("[bench] sweep", sweep[-1])
        del Li

    # ---- lognormal expert popularity (the planner workload of the thakicloud.com post) -------
    lognormal = None
    if not args.no_sweep:
        c = W.LOGNORMAL
        dl = M.Dims.make(c["R"], c["E"], B, c["S"], c["K"], H)
        Ll = MoonEPLayer(dl, training=False)
        # the same workload under the low-migration plan rule (plan only: the rows differ, the
        # dispatch and combine bytes do not)
        dlo = M.Dims.make(c["R"], c["E"], B, c["S"], c["K"], H, plan_rule="lowmig")
        Llo = MoonEPLayer(dlo, training=False)
        xl = torch.randn((c["R"], c["S"], H), device=dev).to(torch.bfloat16)
        with open(os.path.join(ROOT, "tests", "golden", "lognormal_table1.json")) as f:
            post = {row[0]: row for row in json.load(f)["rows"]}
        lognormal = []
        for sg in c["sigmas"]:
            tkl, gl = W.lognormal_routing(c["R"], c["S"], c["E"], c["K"], sg)
            tkd, gd = torch.from_numpy(np.array(tkl)).to(dev), torch.from_numpy(gl).to(dev)
            T4 = Timer(torch)
            for it in range(4):
                T4.run("plan", lambda: Ll.plan(tkd))
                T4.run("dispatch", lambda: Ll.dispatch(xl))
                T4.run("combine", lambda: Ll.combine(gd))
                if it == 0:
                    torch.cuda.synchronize()
                    T4.clear()
            for it in range(4):
                T4.run("plan_lowmig", lambda: Llo.plan(tkd))
            torch.cuda.synchronize()
            m4 = T4.avg_ms()
            s4 = Ll.stats.cpu().numpy()
            s5 = Llo.stats.cpu().numpy()
            cap = c["S"] * c["K"]
            rows_l = c["R"] * cap
            dcb = 2 * (c["R"] * c["S"] * H * 2 + rows_l * H * 2) + 12.0 * rows_l
            p = post.get(sg)
            lognormal.append({
                "sigma": sg, "baseline_peak_load": int(s4[8]), "baseline_min_load": int(s4[9]),
                "peak_over_mean": round(int(s4[8]) / cap, 3), "moonep_peak_over_mean": 1.0,
                "migrated_pct": round(100.0 * int(s4[5]) / rows_l, 2),
                "migration_bound_pct": round(100.0 * int(s4[6]) / rows_l, 2),
                "copies": int(s4[1]), "fallback": int(s4[3]), "plan_us": round(m4["plan"] * 1e3, 1),
                "lowmig": {"migrated_pct": round(100.0 * int(s5[5]) / rows_l, 2), "copies": int(s5[1]),
                           "fallback": int(s5[3]), "plan_us": round(m4["plan_lowmig"] * 1e3, 1)},
                "dc_GBps": round(dcb / ((m4["dispatch"] + m4["combine"]) / 1e3) / 1e9, 1),
                "post_table1": None if p is None else {"peak_over_mean": p[3], "migrated_pct": p[5],
                                                       "copy_slots": p[6]},
            })
            log("[bench] lognormal", lognormal[-1])
        del Ll, Llo, xl

    # ---- zero-copy ablation: the staged baseline (arrival-order copy + sort-copy) ------------
    ablation = None
    if not args.no_sweep:
        stage = torch.empty_like(L.recv)
        T3 = Timer(torch)
        for it in range(4):
            T3.run("dispatch", lambda: L.dispatch(x))
            T3.run("dispatch_staged", lambda: M.moonep_dispatch_staged(d, L.dest, x, None, stage, L.recv))
            T3.run("combine", lambda: L.combine(g))
            T3.run("combine_staged", lambda: M.moonep_combine_staged(d, L.dest, L.y, g, stage, L.out))
            if it == 0:
                torch.cuda.synchronize()
                T3.clear()
        torch.cuda.synchronize()
        m3 = T3.avg_ms()
        del stage
        Mr = R * S * K
        xb_, rb_ = R * S * H * 2, Mr * H * 2
        moved_d = (xb_ + rb_) + (4.0 * Mr + 2 * rb_)            # arrival-order copy, then the sort-copy
        moved_c = (4.0 * Mr + 2 * rb_) + (rb_ + 4.0 * Mr + xb_)  # gather back, then the reduction
        alg = work["dispatch"][1] + work["combine"][1]
        ablation = {
            "fused_ms": round(m3["dispatch"] + m3["combine"], 4),
            "staged_ms": round(m3["dispatch_staged"] + m3["combine_staged"], 4),
            "dispatch_ms": round(m3["dispatch"], 4), "dispatch_staged_ms": round(m3["dispatch_staged"], 4),
            "combine_ms": round(m3["combine"], 4), "combine_staged_ms": round(m3["combine_staged"], 4),
            "algorithmic_GB": round(alg / 1e9, 3), "staged_moved_GB": round((moved_d + moved_c) / 1e9, 3),
            "fused_GBps": round(alg / ((m3["dispatch"] + m3["combine"]) / 1e3) / 1e9, 1),
            "staged_moved_GBps": round((moved_d + moved_c) / ((m3["dispatch_staged"] + m3["combine_staged"]) / 1e3)
                                       / 1e9, 1),
            "speedup": round((m3["dispatch_staged"] + m3["combine_staged"]) / (m3["dispatch"] + m3["combine"]), 3),
        }
        log("[bench] zero-copy ablation", ablation)

    # ---- process-global prefetch pool: slot memory across depth, and its re-prefetch cost ----
    from balanced_token_dispatch_moonep_amd.layer import MoonEPPool, stack_slot_bytes
    pool = {
        "per_set_GB": round(MoonEPPool.nbytes(R, B, H, I, training=True)["total"] / 1e9, 3),
        "layers": {str(n): {"pooled_GB": round(stack_slot_bytes(R, B, H, I, n, True, True) / 1e9, 3),
                            "per_layer_GB": round(stack_slot_bytes(R, B, H, I, n, False, True) / 1e9, 3)}
                   for n in (1, 8, 64)},
        "re_prefetch_ms_per_layer": round(ms["prefetch"], 4),
    }
    if not args.no_sweep:
        pool["measured"] = measured_stack_peaks(torch, M, W, MoonEPLayer, MoonEPPool, stack_slot_bytes,
                                                cfg, dev, log)

    # ---- practical HBM ceilings on this GPU (context only: 8 TB/s stays the denominator) ------
    # the library's weight prefetch is a plain 16-byte copy; torch's copy and fill show what the
    # runtime's own streaming kernels reach on the same device
    def _rate(fn, nbytes, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return round(nbytes / (a.elapsed_time(b) / reps / 1e3) / 1e9, 1)

    nb = 1 << 32
    src_buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst_buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    hbm_context = {
        "prefetch_copy_GBps": rooflines["prefetch"]["achieved"],
        "torch_copy_GBps": _rate(lambda: dst_buf.copy_(src_buf), 2 * nb),
        "torch_fill_GBps": _rate(lambda: dst_buf.fill_(7), nb),
        "buffer_GiB": nb >> 30,
    }
    del src_buf, dst_buf
    log("[bench] hbm context", hbm_context)

    # ---- the vendor library's dense bf16 product on the gate/up shape (context only: 2.5 PFLOP/s
    # stays the denominator).  Dense rows (no grouping, no padding): R*S tokens x H @ H x 2I.
    mm_a = torch.randn((R * S, H), dtype=torch.bfloat16, device=dev)
    mm_b = torch.randn((H, 2 * I), dtype=torch.bfloat16, device=dev)
    mm_flop = 2.0 * R * S * H * 2 * I
    mm_gflops = _rate(lambda: mm_a @ mm_b, mm_flop)   # GFLOP/s (the helper divides by 1e9)
    del mm_a, mm_b
    # ... and its batched product on the weight-gradient shape: per expert, H x (rows) @ (rows) x 2I
    # with rows = one expert's mean share of the receive buffer and float32 output, as dW13 writes
    # (64 experts' worth; operands contiguous)
    nb_t, kr = 64, max(32, (R * S * K) // (E + R * B))
    bm_a = torch.randn((nb_t, H, kr), dtype=torch.bfloat16, device=dev).contiguous()
    bm_b = torch.randn((nb_t, kr, 2 * I), dtype=torch.bfloat16, device=dev).contiguous()
    bm_gflops = _rate(lambda: torch.bmm(bm_a, bm_b, out_dtype=torch.float32), 2.0 * nb_t * H * kr * 2 * I)
    del bm_a, bm_b
    torch.cuda.empty_cache()
    mfma_context = {
        "torch_bf16_matmul_TFLOPs": round(mm_gflops / 1e3, 1),
        "shape": f"{R * S}x{H} @ {H}x{2 * I}",
        "frac_of_peak": round(mm_gflops / 1e3 / MFMA_BF16_PEAK_TFLOPS, 4),
        "gemm_gate_up_vs_it": round(rooflines["gemm_gate_up"]["achieved"] / (mm_gflops / 1e3), 4),
        "torch_bf16_bmm_fp32_out_TFLOPs": round(bm_gflops / 1e3, 1),
        "bmm_shape": f"{nb_t} x ({H}x{kr} @ {kr}x{2 * I}), float32 out",
        "gemm_dw13_vs_it": round(rooflines["gemm_dw13"]["achieved"] / (bm_gflops / 1e3), 4),
    }
    log("[bench] mfma context", mfma_context)

    # ---- CPU oracle baseline on a bounded sample of the same workload ----------------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, args.cpu_tokens, args.cpu_groups, log)

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
        "gemm_fwd_TFLOPs": round(fwd_tflops, 1),
        "gemm_bwd_TFLOPs": round(bwd_tflops, 1),
        "roofline": roofline,
        "rooflines": rooflines,
        "sweep": sweep,
        "zero_copy_ablation": ablation,
        "lognormal_planner": lognormal,
        "prefetch_pool": pool,
        "hbm_context": hbm_context,
        "mfma_context": mfma_context,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def measured_stack_peaks(torch, M, W, MoonEPLayer, MoonEPPool, stack_slot_bytes, cfg, dev, log,
                         depths=(1, 2, 4)):
    """Device memory peak of a training stack of n layers (forward through all, backward in
    reverse), with one prefetch pool for all layers or slots and reduce buffers per layer.
    Measured with torch's allocator statistics at a shape whose per-layer buffers are small
    (E=16 experts, S=512 tokens per rank) while the slots and reduce buffers keep their full
    size (R, B, H, I as the benchmarked layer), so the pool is what the depth changes."""
    R, B, H, I, K = cfg.R, cfg.B, cfg.H, cfg.I, cfg.K
    E, S = 2 * R, 512
    c = cfg.with_(E=E, S=S, lam=1.0, maxvio=None)
    topk, gates, _ = W.routing_for(c)
    tk, g = torch.from_numpy(topk).to(dev), torch.from_numpy(gates).to(dev)
    x = torch.randn((R, S, H), device=dev).to(torch.bfloat16)
    dout = torch.randn((R, S, H), device=dev).to(torch.bfloat16)
    d = M.Dims.make(R, E, B, S, K, H, I, training=True)
    out = {"shape": f"R{R} E{E} B{B} S{S} K{K} H{H} I{I}, training", "depths": {}}

    def peak_of(n, pooled):
        # everything the stack allocates is local to this call, so it is freed on return
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        p = MoonEPPool(R, B, H, I, training=True, device=dev) if pooled else None
        stack = [MoonEPLayer(d, *W.expert_weights_torch(E, H, I, 50 + l, dev), training=True, pool=p)
                 for l in range(n)]
        h = x
        for layer in stack:
            h = layer.forward(h, tk, g).clone()
        dh = dout
        for layer in reversed(stack):
            dh = layer.backward(dh, g).clone()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    for n in depths:
        res = {}
        for pooled in (True, False):
            gc.collect()
            torch.cuda.empty_cache()
            res["pooled_peak_GB" if pooled else "per_layer_peak_GB"] = round(peak_of(n, pooled) / 1e9, 3)
        res["measured_saving_GB"] = round(res["per_layer_peak_GB"] - res["pooled_peak_GB"], 3)
        res["formula_saving_GB"] = round((stack_slot_bytes(R, B, H, I, n, False, True) -
                                          stack_slot_bytes(R, B, H, I, n, True, True)) / 1e9, 3)
        out["depths"][str(n)] = res
        log("[bench] stack peak", n, res)
    torch.cuda.empty_cache()
    return out


def algorithmic_work(cfg, st, cu, dst, topk):
    """Per timed call: (bound, algorithmic bytes or flops, algorithmic HBM bytes, per-launch text).

    Bytes count what the method must move (each operand read once, each result written once);
    flops count real rows only (2 per multiply-add), never padding."""
    import numpy as np
    R, E, B, S, K, H, I = cfg.R, cfg.E, cfg.B, cfg.S, cfg.K, cfg.H, cfg.I
    Mr = R * S * K
    xbytes, rbytes, NW = R * S * H * 2, Mr * H * 2, 3 * H * I
    n_slot = int(st[2])
    # expert of each slot replica (slot rows of cu_seqlens; the expert of their first row via dest)
    row_expert = np.full(Mr, -1, dtype=np.int64)
    row_expert[dst] = topk.ravel()
    reps = {}
    for q in range(R):
        for j in range(B):
            lo, hi = cu[q, E + j], cu[q, E + j + 1]
            if hi > lo:
                e = int(row_expert[q * S * K + lo])
                reps[e] = reps.get(e, 0) + 1
    rg = float(sum((8 + 8 * n) * NW for n in reps.values()))
    mhi = float(Mr) * H * I
    # GEMM operand bytes (each operand and result once): A rows, the weights of every group, out
    wgroups = E + n_slot + int(st[3])
    gem = {
        "gemm_gate_up": (4 * mhi, Mr * H * 2 + wgroups * H * 2 * I * 2 + Mr * I * 2 * 3),
        "gemm_down": (2 * mhi, Mr * I * 2 + wgroups * I * H * 2 + Mr * H * 2),
        "gemm_dact": (2 * mhi, Mr * H * 2 + wgroups * I * H * 2 + Mr * 2 * I * 2 * 2),
        "gemm_dx": (4 * mhi, Mr * 2 * I * 2 + wgroups * H * 2 * I * 2 + Mr * H * 2),
        "gemm_dw2": (2 * mhi, Mr * I * 2 + Mr * H * 2 + (E + n_slot) * I * H * 4),
        "gemm_dw13": (4 * mhi, Mr * H * 2 + Mr * 2 * I * 2 + (E + n_slot) * H * 2 * I * 4),
    }
    work = {
        "plan": ("hbm", 8.0 * Mr, 8.0 * Mr, f"topk read + dest write, {Mr} pairs (3 kernels)"),
        "prefetch": ("hbm", 2.0 * n_slot * NW * 2, 2.0 * n_slot * NW * 2,
                     f"{n_slot} slot replicas x 2 x {NW} bf16 weights (read + write)"),
        "dispatch": ("hbm", xbytes + rbytes + 4.0 * Mr, xbytes + rbytes + 4.0 * Mr,
                     f"{R * S} rows read once, {Mr} rows written, {Mr} dest"),
        "combine": ("hbm", rbytes + 8.0 * Mr + xbytes, rbytes + 8.0 * Mr + xbytes,
                    f"{Mr} rows read, {R * S} rows written, dest + gates"),
        "dispatch_bwd": ("hbm", xbytes + rbytes + 8.0 * Mr, xbytes + rbytes + 8.0 * Mr,
                         f"{R * S} rows read once, {Mr} scaled rows written, dest + gates"),
        "combine_bwd": ("hbm", rbytes + 4.0 * Mr + xbytes, rbytes + 4.0 * Mr + xbytes,
                        f"{Mr} rows read, {R * S} rows written, dest"),
        "reduce_grad": ("hbm", rg, rg, f"{len(reps)} replicated experts, {sum(reps.values())} slot replicas, "
                                       f"(8 + 8n) x {NW} bytes each"),
    }
    for k, (fl, by) in gem.items():
        work[k] = ("mfma", fl, float(by), f"{fl / mhi:.0f} x M*H*I flops, M={Mr} real rows, H={H}, I={I}")
    return work


def roofline_of(name, w, ms):
    bound, amount = w[0], w[1]
    t = ms / 1e3
    if bound == "hbm":
        ach = amount / t / 1e9 if t > 0 else 0.0
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "ms": round(ms, 4), "bytes": amount}
    ach = amount / t / 1e12 if t > 0 else 0.0
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "ms": round(ms, 4), "flops": amount,
            "operand_bytes": w[2]}


def _code_only(text):
    """C++ source without comments and blank lines (string literals in these sources hold no
    comment markers), so that a comment edit does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def _sources_digest(call):
    """Digest of the code (comments excluded) of the call's kernel sources."""
    import hashlib
    csrc = os.path.join(ROOT, "balanced_token_dispatch_moonep_amd", "csrc")
    files = KERNEL_SOURCES.get(call, ("gemm.hip",)) + ("common.h",)
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def stored_of(path, call, field):
    """A per-call figure stored by a counter reducer, or None when none is stored for the
    call's kernel as it is now built (digest of its sources, comments excluded)."""
    try:
        with open(path) as f:
            rec = json.load(f).get(call)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources") != _sources_digest(call):
        return None
    return rec.get(field)


def traffic_of(call, algorithmic_bytes):
    """HBM bytes per launch of the call's kernel from the stored rocprofv3 FETCH_SIZE / WRITE_SIZE
    counts (scaled by a copy kernel of known size), or None when none are stored for the kernel
    as it is now built."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(call)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources") != _sources_digest(call):
        return None
    return rec.get("hbm_bytes_per_launch")


def _kernel_call(kname):
    """The timed call whose kernel a rocprofv3 kernel name is, or None."""
    n = kname[5:] if kname.startswith("void ") else kname
    for call, k in KERNEL_NAMES.items():
        if n.startswith(k + "("):
            return call
    return None


def _pmc_per_dispatch(d, counter):
    """Mean per dispatch of one counter, per kernel name, from a rocprofv3 -f csv output tree."""
    import csv
    import glob
    tot = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                tot[key] = tot.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (k, _), v in tot.items():
        per.setdefault(k, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}


def write_traffic(fetch_dir, write_dir, bench_json):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every timed kernel, scaled by what the same
    counters read for the weight prefetch, a plain copy of known size."""
    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    run = json.loads(line)
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")
    calls = {}
    for k in set(fetch) | set(write):
        c = _kernel_call(k)
        if c:
            calls[c] = k
    if "prefetch" not in calls:
        print("no prefetch kernel in the counter runs: nothing to calibrate against", file=sys.stderr)
        return 1
    copy_bytes = run["rooflines"]["prefetch"]["bytes"] / 2       # read once, written once
    kf = copy_bytes / (fetch[calls["prefetch"]][0] * 1024.0)
    kw = copy_bytes / (write[calls["prefetch"]][0] * 1024.0)
    out = {"_calibration": {"copy_kernel": KERNEL_NAMES["prefetch"], "copy_bytes_each_way": copy_bytes,
                            "fetch_factor": round(kf, 4), "write_factor": round(kw, 4),
                            "workload": run["config"]}}
    rows = []
    for c in KERNEL_NAMES:
        if c not in calls:
            continue
        k = calls[c]
        fb = fetch.get(k, (0.0, 0))[0] * 1024.0 * kf
        wb = write.get(k, (0.0, 0))[0] * 1024.0 * kw
        r = run["rooflines"].get(c, {})
        alg = r.get("bytes", r.get("operand_bytes"))
        out[c] = {"kernel": KERNEL_NAMES[c], "fetch_bytes": round(fb), "write_bytes": round(wb),
                  "hbm_bytes_per_launch": round(fb + wb), "sources": _sources_digest(c),
                  "dispatches": fetch.get(k, (0.0, 0))[1]}
        rows.append(f"| `{KERNEL_NAMES[c]}` | {c} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {(fb + wb) / 1e9:.3f} | "
                    + (f"{alg / 1e9:.3f} | {(fb + wb) / alg:.2f} |" if alg else "— | — |"))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"Copy calibration: `{KERNEL_NAMES['prefetch']}` moves {copy_bytes / 1e9:.3f} GB each way; "
          f"FETCH_SIZE x {kf:.4f}, WRITE_SIZE x {kw:.4f}.\n")
    print("| kernel | call | fetch GB | write GB | HBM GB / launch | algorithmic GB | ratio |")
    print("|---|---|---:|---:|---:|---:|---:|")
    print("\n".join(rows))
    return 0


def _kernel_durations(d):
    """Mean duration (ns) per kernel name from a rocprofv3 kernel_trace.csv tree."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                per.setdefault(row["Kernel_Name"], []).append(
                    int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def write_mfma(pmc_dir, bench_json):
    """Matrix-core busy fraction of every timed GEMM kernel.

    SQ_VALU_MFMA_BUSY_CYCLES is counted per SIMD and GRBM_GUI_ACTIVE per XCD; rocprofv3 sums
    each over its instances.  busy = MFMA busy cycles / (GUI-active cycles of one XCD x 1024
    SIMDs).  SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 is the bf16 flops the matrix cores executed
    (padding included).  The implied shader clock is one XCD's GUI-active cycles over the
    kernel's traced duration."""
    with open(bench_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    run = json.loads(line)
    busy = _pmc_per_dispatch(pmc_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    mops = _pmc_per_dispatch(pmc_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    grbm = _pmc_per_dispatch(pmc_dir, "GRBM_GUI_ACTIVE")
    dur = _kernel_durations(pmc_dir)
    out = {"_method": {"busy": "sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)",
                       "executed_flops": "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512",
                       "clock": "GRBM_GUI_ACTIVE / 8 / traced duration", "workload": run["config"]}}
    rows = []
    for c, kname in KERNEL_NAMES.items():
        if not c.startswith("gemm_"):
            continue
        k = next((n for n in busy if _kernel_call(n) == c), None)
        if k is None or k not in grbm:
            continue
        cyc = grbm[k][0] / XCDS
        frac = busy[k][0] / (cyc * SIMDS)
        exe = mops.get(k, (0.0, 0))[0] * 512.0
        alg = run["rooflines"].get(c, {}).get("flops")
        ns = dur.get(k)
        ghz = cyc / ns if ns else None
        out[c] = {"kernel": kname, "mfma_busy_frac": round(frac, 4), "gui_cycles": round(cyc),
                  "executed_flops": exe, "algorithmic_flops": alg,
                  "executed_over_algorithmic": round(exe / alg, 4) if alg else None,
                  "traced_ms": round(ns / 1e6, 4) if ns else None,
                  "clock_GHz": round(ghz, 3) if ghz else None,
                  "sources": _sources_digest(c), "dispatches": busy[k][1]}
        rows.append(f"| `{kname}` | {c} | {frac:.3f} | {exe / 1e12:.2f} | "
                    + (f"{alg / 1e12:.2f} | {exe / alg:.3f} | " if alg else "— | — | ")
                    + (f"{ns / 1e6:.2f} | {ghz:.2f} |" if ns else "— | — |"))
    with open(MFMA_FILE, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print("| kernel | call | MFMA busy | executed TFLOP | algorithmic TFLOP | executed / algorithmic | "
          "traced ms | implied clock GHz |")
    print("|---|---|---:|---:|---:|---:|---:|---:|")
    print("\n".join(rows))
    return 0


def l2_rows(dir1, dir2):
    """Per GEMM call: mean traced ms, L2 hit rate, reads beyond L2 (128-byte requests), their mean
    latency (TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, in L2 cycles), the writes' mean latency and the
    tag stalls, from two rocprofv3 --pmc runs with --kernel-trace."""
    cnt = {c: _pmc_per_dispatch(dir1 if c in ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum",
                                              "TCC_EA0_RDREQ_LEVEL_sum") else dir2, c)
           for c in ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_LEVEL_sum",
                     "TCC_TAG_STALL_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_LEVEL_sum")}
    dur = _kernel_durations(dir1)
    out = []
    for call, kname in KERNEL_NAMES.items():
        if not call.startswith("gemm_"):
            continue
        k = next((n for n in cnt["TCC_HIT_sum"] if _kernel_call(n) == call), None)
        if k is None or any(k not in cnt[c] for c in cnt):
            continue
        v = {c: cnt[c][k][0] for c in cnt}
        rd, wr = v["TCC_EA0_RDREQ_sum"], v["TCC_EA0_WRREQ_sum"]
        ms = dur.get(k, 0.0) / 1e6
        out.append({"call": call, "kernel": kname, "ms": ms,
                    "hit": v["TCC_HIT_sum"] / max(v["TCC_HIT_sum"] + v["TCC_MISS_sum"], 1.0),
                    "reads": rd, "read_GB": rd * 128 / 1e9,
                    "read_latency": v["TCC_EA0_RDREQ_LEVEL_sum"] / rd if rd else None,
                    "write_latency": v["TCC_EA0_WRREQ_LEVEL_sum"] / wr if wr else None,
                    "tag_stall": v["TCC_TAG_STALL_sum"]})
    return out


def print_l2(dir1, dir2):
    print("| kernel | call | ms | L2 hit rate | reads beyond L2 (128 B) | rate | mean miss latency | "
          "mean write latency | tag stalls |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|")
    for r in l2_rows(dir1, dir2):
        rate = f"{r['read_GB'] / r['ms']:.2f} TB/s" if r["ms"] else "—"
        rl = f"{r['read_latency']:.0f} cycles" if r["read_latency"] is not None else "—"
        wl = f"{r['write_latency']:.0f} cycles" if r["write_latency"] is not None else "—"
        print(f"| `{r['kernel']}` | {r['call']} | {r['ms']:.2f} | {r['hit'] * 100:.0f}% | "
              f"{r['reads']:.3g} ({r['read_GB']:.1f} GB) | {rate} | {rl} | {wl} | {r['tag_stall']:.2g} |")
    return 0


def print_stats(d):
    """Markdown table of rocprofv3's kernel_stats.csv (durations in microseconds)."""
    import csv
    import glob
    fs = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not fs:
        print(f"no kernel_stats.csv under {d}", file=sys.stderr)
        return 1
    print("| kernel | call | calls | avg us | min us | max us | total ms |")
    print("|---|---|---:|---:|---:|---:|---:|")
    with open(fs[0]) as fh:
        for row in csv.DictReader(fh):
            name = row["Name"]
            short = name if len(name) <= 90 else name[:87] + "..."
            print(f"| `{short}` | {_kernel_call(name) or ''} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
                  f"{float(row['MinNs']) / 1e3:.1f} | {float(row['MaxNs']) / 1e3:.1f} | "
                  f"{float(row['TotalDurationNs']) / 1e6:.2f} |")
    return 0


def group_stats(cu):
    """GEMM groups of a plan (rank, weight row) with rows, their 256-row tiles and the padding share."""
    import numpy as np
    rows = np.diff(np.asarray(cu, dtype=np.int64), axis=1)
    nz = rows[rows > 0]
    tiles = int(((nz + 255) // 256).sum())
    return {"groups": int(nz.size), "row_tiles": tiles,
            "padding_frac": round(1.0 - float(nz.sum()) / (tiles * 256), 4) if tiles else 0.0}


def sweep_entry(c, tk, lam, s, m, w, kind, cu=None):
    import numpy as np
    Mr = c.R * c.S * c.K
    Lx = np.bincount(tk.ravel(), minlength=c.E).astype(np.float64)
    ent = {"variant": kind, "B": c.B,
           "maxvio": round(float((Lx.max() - Lx.mean()) / Lx.mean()), 3), "lambda": round(lam, 4),
           "replicas": int(s[1]), "slot_replicas": int(s[2]), "fallback_replicas": int(s[3]),
           "fallback_rows": int(s[4]), "migrated_frac": round(int(s[5]) / Mr, 4),
           "migration_bound_frac": round(int(s[6]) / Mr, 4),
           "rank_peak_over_mean": round(int(s[8]) / (c.S * c.K), 4),
           "plan_us": round(m["plan"] * 1e3, 1), "prefetch_ms": round(m["prefetch"], 4),
           "dispatch_ms": round(m["dispatch"], 4), "combine_ms": round(m["combine"], 4),
           "dc_GBps": round((w["dispatch"][1] + w["combine"][1]) / ((m["dispatch"] + m["combine"]) / 1e3) / 1e9, 1)}
    if cu is not None:
        ent.update(group_stats(cu))
    fwd = [k for k in ("gemm_gate_up", "gemm_down") if k in m]
    if fwd:
        fl = sum(w[k][1] for k in fwd)
        t = sum(m[k] for k in fwd)
    else:
        fl = w["gemm_gate_up"][1] + w["gemm_down"][1]
        t = m["ffn_fwd"]
    ent["gemm_fwd_ms"] = round(t, 3)
    ent["gemm_fwd_TFLOPs"] = round(fl / (t / 1e3) / 1e12, 1)
    bwd = [k for k in ("gemm_dact", "gemm_dx", "gemm_dw2", "gemm_dw13") if k in m]
    if bwd:
        flb = sum(w[k][1] for k in bwd)
        tb = sum(m[k] for k in bwd)
        ent["gemm_bwd_ms"] = round(tb, 3)
        ent["gemm_bwd_TFLOPs"] = round(flb / (tb / 1e3) / 1e12, 1)
        ent["dc_bwd_GBps"] = round((w["dispatch_bwd"][1] + w["combine_bwd"][1]) /
                                   ((m["dispatch_bwd"] + m["combine_bwd"]) / 1e3) / 1e9, 1)
        ent["reduce_grad_ms"] = round(m["reduce_grad"], 4)
    return ent


def cpu_baseline(cfg, tokens, ngroups, log):
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
    grp = O.groups(plan)[:ngroups]
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
                  f"FFN forward on {len(grp)} groups in float64 (ffn_TFLOPs)",
        "plan_s": round(t1 - t0, 3),
        "dispatch_s": round(t2 - t1, 3),
        "combine_s": round(t3 - t2, 3),
        "ffn_TFLOPs": round(flops / (t5 - t4) / 1e12, 4),
        "threads": os.environ.get("OMP_NUM_THREADS", str(cores)),
        "cpu_model": _cpu_model() or platform.processor(),
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
    return ""


if __name__ == "__main__":
    sys.exit(main())
