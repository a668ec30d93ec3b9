"""GPU parity of weight prefetch, the grouped SwiGLU GEMM (forward and backward) and
reduce_grad against the CPU oracle.

Tolerance: relative Frobenius error <= 2e-2 for GEMM outputs and gradients (bf16
inputs and outputs, fp32 accumulation, against a float64 oracle); prefetched slots
and the permuted rows are bit-exact.
"""
import numpy as np
import pytest
import torch

import balanced_token_dispatch_moonep_amd as M
from balanced_token_dispatch_moonep_amd.layer import MoonEPLayer, MoonEPPool
import oracle as O
import workload as W

from gpu_util import (DEV, say, dims_of, i32, f32, bf16_from_bits, bits_of, f64_of,
                      assert_plan_parity, rel_fro, max_row_rel)

pytestmark = pytest.mark.gpu
TOL = 2e-2

# several 256x256 tiles per group with ragged tails; I = 320 is not a multiple of 128,
# so the gate/up column tiles and the dA / dW column tiles are partial too
MID = W.Config("mid", R=4, E=16, B=4, S=512, K=4, H=512, I=320, dtype="bf16", lam=1.0, seed=2)


def _setup(cfg, B=None, training=False):
    topk, gates, _ = W.routing_for(cfg)
    xb = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    w13f, w2f = W.expert_weights_np(cfg.E, cfg.H, cfg.I, cfg.seed)
    wb13, wb2 = W.bf16_bits(w13f), W.bf16_bits(w2f)
    d = dims_of(cfg, B=B, training=training, f32_rows=False)
    plan, dest, _ = assert_plan_parity(d, topk, training=training)
    layer = MoonEPLayer(d, w13=bf16_from_bits(wb13), w2=bf16_from_bits(wb2), training=training)
    return topk, gates, xb, wb13, wb2, d, plan, dest, layer


@pytest.mark.parametrize("B", [4, 2, 0])
def test_forward_mid(B):
    _forward_check(MID.with_(B=B))


# tiles cut in every dimension: H and I not multiples of the 256-wide (128 for gate/up) tiles
RAGGED = [dict(H=576, I=192), dict(H=320, I=448, K=3, S=300)]


@pytest.mark.parametrize("over", RAGGED, ids=lambda o: "-".join(f"{k}{v}" for k, v in o.items()))
def test_forward_ragged_tiles(over):
    _forward_check(MID.with_(**over))


@pytest.mark.parametrize("over", RAGGED, ids=lambda o: "-".join(f"{k}{v}" for k, v in o.items()))
def test_backward_ragged_tiles(over):
    _backward_check(MID.with_(**over))


def _forward_check(cfg):
    B = cfg.B
    topk, gates, xb, wb13, wb2, d, plan, dest, layer = _setup(cfg)
    say("forward", cfg, "replicas", len(plan.entries),
        "fallback", sum(1 for e in plan.entries if e.w < cfg.E))
    out = layer.forward(bf16_from_bits(xb), i32(topk), f32(gates))
    torch.cuda.synchronize()
    recv = O.dispatch(dest, xb)
    assert bits_of(layer.recv).tobytes() == recv.tobytes()
    s13, s2 = O.prefetch(plan, wb13, wb2)
    if B:
        for en in plan.entries:
            if en.w >= cfg.E:
                assert np.array_equal(bits_of(layer.w13_slot[en.q, en.j]), s13[en.q, en.j])
                assert np.array_equal(bits_of(layer.w2_slot[en.q, en.j]), s2[en.q, en.j])
    gu, act, y = O.ffn_forward(plan, recv, wb13, wb2, s13, s2)
    for name, got, ref in (("gu", layer.gu, gu), ("act", layer.act, act), ("y", layer.y, y)):
        e = rel_fro(f64_of(got), ref)
        say(f"  {name} rel fro {e:.3e}")
        assert e <= TOL
    for (q, w, row0, rows, kind, idx) in O.groups(plan):
        assert rel_fro(f64_of(layer.y[row0:row0 + rows]), y[row0:row0 + rows]) <= TOL, (q, w, kind)
    ref = O.combine(dest, y, gates)
    assert max_row_rel(f64_of(out), ref) <= TOL
    # the plan-free definition (duplicates and fallback do not change the result)
    direct = O.moe_direct(xb, topk, gates, wb13, wb2)
    e = rel_fro(f64_of(out), direct)
    say(f"  out vs direct rel fro {e:.3e}")
    assert e <= TOL


def test_forward_deterministic():
    topk, gates, xb, wb13, wb2, d, plan, dest, layer = _setup(MID)
    x, tk, g = bf16_from_bits(xb), i32(topk), f32(gates)
    first = layer.forward(x, tk, g).clone()
    y1 = layer.y.clone()
    for _ in range(2):
        assert torch.equal(layer.forward(x, tk, g).view(torch.int16), first.view(torch.int16))
        assert torch.equal(layer.y.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("B", [4, 2, 0])
def test_backward_mid(B):
    _backward_check(MID.with_(B=B))


# Many groups that end in a tail of at most 128 rows: row tiles that are mostly padding rows
# (loaded as zeros), whose outputs must not be stored; the plan must hold such tails for the case
# to exercise them
WIDE = MID.with_(H=512, I=512, S=400, seed=6)


def _short_tails(cfg):
    topk, _, _ = W.routing_for(cfg)
    plan = O.make_plan(topk, cfg.E, cfg.B)
    rows = np.diff(np.asarray(plan.cu), axis=1).ravel()
    return int(np.sum((rows % 256 > 0) & (rows % 256 <= 128)))


@pytest.mark.parametrize("B", [4, 0])
def test_forward_backward_short_tails(B):
    cfg = WIDE.with_(B=B)
    assert _short_tails(cfg) >= 4
    _forward_check(cfg)
    _backward_check(cfg)


def _random_cfgs(n=4, seed=11):
    """Seeded random small layers: rank counts, slots (including none, so fallback targets with
    several row segments), top-k, ragged H and I, and skew all vary."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([2, 4, 8]))
        E = R * int(rng.choice([2, 4]))
        out.append(MID.with_(R=R, E=E, B=int(rng.choice([0, 1, 2, 4])),
                             K=int(rng.integers(1, min(E, 4) + 1)), S=int(rng.choice([96, 200, 333, 512])),
                             H=int(rng.choice([256, 320, 576])), I=int(rng.choice([128, 192, 320])),
                             lam=round(float(rng.uniform(0.0, 2.0)), 3), seed=100 + i))
    return out


@pytest.mark.parametrize("cfg", _random_cfgs(), ids=lambda c: f"R{c.R}E{c.E}B{c.B}K{c.K}S{c.S}H{c.H}I{c.I}")
def test_backward_random_shapes(cfg):
    _backward_check(cfg)


def _backward_check(cfg):
    B = cfg.B
    topk, gates, xb, wb13, wb2, d, plan, dest, layer = _setup(cfg, training=True)
    say("backward", cfg)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    layer.forward(bf16_from_bits(xb), i32(topk), f32(gates))
    dx = layer.backward(bf16_from_bits(dout), f32(gates))
    torch.cuda.synchronize()
    recv = O.dispatch(dest, xb)
    s13, s2 = O.prefetch(plan, wb13, wb2)
    gu, act, y = O.ffn_forward(plan, recv, wb13, wb2, s13, s2)
    dy = O.dispatch(dest, dout, row_scale=gates)
    drecv, dW13, dW2, rb13, rb2 = O.ffn_backward(plan, recv, gu, act, dy, wb13, wb2, s13, s2)
    e = rel_fro(f64_of(layer.drecv), drecv)
    say(f"  drecv rel fro {e:.3e}")
    assert e <= TOL
    dx_ref = O.combine(dest, drecv, None)
    assert rel_fro(f64_of(dx), dx_ref) <= TOL
    O.reduce_grad(plan, dW13, dW2, rb13, rb2)
    g13, g2 = f64_of(layer.dw13), f64_of(layer.dw2)
    e13, e2 = rel_fro(g13, dW13), rel_fro(g2, dW2)
    say(f"  dW13 rel fro {e13:.3e}  dW2 rel fro {e2:.3e}")
    assert e13 <= TOL and e2 <= TOL
    for ex in range(cfg.E):
        if plan.L[ex] > 0:
            assert rel_fro(g13[ex], dW13[ex]) <= TOL, ex
            assert rel_fro(g2[ex], dW2[ex]) <= TOL, ex
        else:
            assert not g13[ex].any() and not g2[ex].any()
    if B:
        assert not layer.dw13_red.any() and not layer.dw2_red.any()
    # plan-free gradients
    rdx, rdW13, rdW2 = O.moe_direct_backward(xb, topk, gates, wb13, wb2, dout)
    assert rel_fro(f64_of(dx), rdx) <= TOL
    assert rel_fro(g13, rdW13) <= TOL and rel_fro(g2, rdW2) <= TOL


def test_side_stream_matches_default_stream():
    """Every call runs on the stream it is handed (torch's current stream, here a second stream of
    default priority): the whole forward and backward there give the default stream's bits."""
    topk, gates, xb, wb13, wb2, d, plan, dest, layer = _setup(MID, training=True)
    x, tk, g = bf16_from_bits(xb), i32(topk), f32(gates)
    dout = bf16_from_bits(W.grad_rows(MID.R, MID.S, MID.H, 5, "bf16"))
    ref = [layer.forward(x, tk, g).clone(), layer.backward(dout, g).clone(), layer.dw13.clone(),
           layer.dw2.clone()]
    torch.cuda.synchronize()
    for t in (layer.y, layer.drecv, layer.dw13, layer.dw2):
        t.fill_(7)                       # stale values cannot pass for results
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = [layer.forward(x, tk, g).clone(), layer.backward(dout, g).clone(), layer.dw13.clone(),
               layer.dw2.clone()]
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_backward_writes_or_accumulates():
    """Without MOONEP_GRAD_ACCUM a second backward on the same batch rewrites the same
    gradients; with it the home gradients double.  Reduce buffers are clean after each step."""
    for accum in (False, True):
        topk, gates, _ = W.routing_for(MID)
        xb = W.hidden_rows(MID.R, MID.S, MID.H, MID.seed, "bf16")
        w13f, w2f = W.expert_weights_np(MID.E, MID.H, MID.I, MID.seed)
        d = M.Dims.make(MID.R, MID.E, MID.B, MID.S, MID.K, MID.H, MID.I, training=True, grad_accum=accum)
        layer = MoonEPLayer(d, w13=bf16_from_bits(W.bf16_bits(w13f)), w2=bf16_from_bits(W.bf16_bits(w2f)),
                            training=True)
        dout = bf16_from_bits(W.grad_rows(MID.R, MID.S, MID.H, 7, "bf16"))
        x, tk, g = bf16_from_bits(xb), i32(topk), f32(gates)
        layer.dw13.fill_(3.0)        # stale content: must be overwritten unless accumulating
        layer.forward(x, tk, g)
        layer.backward(dout, g)
        one13 = layer.dw13.clone()
        one2 = layer.dw2.clone()
        layer.forward(x, tk, g)
        layer.backward(dout, g)
        torch.cuda.synchronize()
        if accum:
            ref = f64_of(one13) - 3.0
            assert rel_fro(f64_of(layer.dw13) - 3.0, 2 * ref) <= 1e-6
        else:
            assert torch.equal(layer.dw13, one13) and torch.equal(layer.dw2, one2)
            assert not bool((layer.dw13 == 3.0).any())
        assert not layer.dw13_red.any()


def test_phases_match_single_call():
    """Each phase flag runs one GEMM kernel; running the phases one call at a time (the weight
    gradients deferred, dW13 before dW2) gives bit-identical results to one call."""
    cfg = MID.with_(B=2)
    topk, gates, xb, wb13, wb2, d, plan, dest, layer = _setup(cfg, training=True)
    dout = bf16_from_bits(W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16"))
    x, tk, g = bf16_from_bits(xb), i32(topk), f32(gates)
    layer.forward(x, tk, g)
    ref = {n: getattr(layer, n).clone() for n in ("gu", "act", "y")}
    M.moonep_dispatch(d, layer.dest, dout, g, layer.dy)
    M.moonep_grouped_ffn_backward(d, layer.ws, layer.cu, layer.recv, layer.gu, layer.act, layer.dy,
                                  layer.w13, layer.w2, layer.w13_slot, layer.w2_slot, layer.drecv,
                                  layer.dw13, layer.dw2, layer.dw13_red, layer.dw2_red)
    ref.update({n: getattr(layer, n).clone() for n in ("drecv", "dw13", "dw2", "dw13_red", "dw2_red")})
    ref["dgu"] = layer.gu.clone()
    for n in ("act", "y", "gu", "drecv", "dw13", "dw2", "dw13_red", "dw2_red"):
        getattr(layer, n).fill_(7.0)                  # stale content everywhere
    for ph in (M.PHASE_GATE_UP, M.PHASE_DOWN):
        M.moonep_grouped_ffn(d.with_flags(d.flags | ph), layer.ws, layer.cu, layer.recv, layer.w13,
                             layer.w2, layer.w13_slot, layer.w2_slot, layer.gu, layer.act, layer.y)
    torch.cuda.synchronize()
    for n in ("gu", "act", "y"):
        assert torch.equal(getattr(layer, n).view(torch.int16), ref[n].view(torch.int16)), n
    for ph in (M.PHASE_DACT, M.PHASE_DX, M.PHASE_DW13, M.PHASE_DW2):
        M.moonep_grouped_ffn_backward(d.with_flags(d.flags | ph), layer.ws, layer.cu, layer.recv, layer.gu,
                                      layer.act, layer.dy, layer.w13, layer.w2, layer.w13_slot, layer.w2_slot,
                                      layer.drecv, layer.dw13, layer.dw2, layer.dw13_red, layer.dw2_red)
    torch.cuda.synchronize()
    assert torch.equal(layer.gu.view(torch.int16), ref["dgu"].view(torch.int16))
    assert torch.equal(layer.drecv.view(torch.int16), ref["drecv"].view(torch.int16))
    for n in ("dw13", "dw2"):
        assert torch.equal(getattr(layer, n), ref[n]), n
    for en in plan.entries:                           # used reduce slots; the others are untouched
        if en.w >= cfg.E:
            assert torch.equal(layer.dw13_red[en.q, en.j], ref["dw13_red"][en.q, en.j])
            assert torch.equal(layer.dw2_red[en.q, en.j], ref["dw2_red"][en.q, en.j])
    # only the selected phase runs
    layer.y.fill_(7.0)
    M.moonep_grouped_ffn(d.with_flags(d.flags | M.PHASE_GATE_UP), layer.ws, layer.cu, layer.recv, layer.w13,
                         layer.w2, layer.w13_slot, layer.w2_slot, layer.gu, layer.act, layer.y)
    torch.cuda.synchronize()
    assert bool((layer.y == 7.0).all())


def test_tiny_layer_f32_rows():
    """Tiny configuration: fp32 token rows for dispatch/combine, bf16 expert GEMM."""
    cfg = W.CONFIGS["tiny"]
    topk, gates, _ = W.routing_for(cfg)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "f32")
    w13f, w2f = W.expert_weights_np(cfg.E, cfg.H, cfg.I, cfg.seed)
    wb13, wb2 = W.bf16_bits(w13f), W.bf16_bits(w2f)
    d32 = dims_of(cfg, f32_rows=True)
    dbf = dims_of(cfg, f32_rows=False)
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d32, topk)
    recv32 = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.float32, device=DEV)
    M.moonep_dispatch(d32, dd, f32(x), None, recv32)
    recv = recv32.to(torch.bfloat16)                  # cast at the bf16 GEMM boundary
    w13, w2 = bf16_from_bits(wb13), bf16_from_bits(wb2)
    s13 = torch.zeros((cfg.R, cfg.B, cfg.H, 2 * cfg.I), dtype=torch.bfloat16, device=DEV)
    s2 = torch.zeros((cfg.R, cfg.B, cfg.I, cfg.H), dtype=torch.bfloat16, device=DEV)
    M.moonep_prefetch(dbf, ws, w13, w2, s13, s2)
    nrows = cfg.R * cfg.C
    act = torch.empty((nrows, cfg.I), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((nrows, cfg.H), dtype=torch.bfloat16, device=DEV)
    M.moonep_grouped_ffn(dbf, ws, cu, recv, w13, w2, s13, s2, None, act, y)
    y32 = y.float()
    out = torch.empty((cfg.R, cfg.S, cfg.H), dtype=torch.float32, device=DEV)
    M.moonep_combine(d32, dd, y32, f32(gates), out)
    torch.cuda.synchronize()
    assert recv32.cpu().numpy().tobytes() == O.dispatch(dest, x).tobytes()
    direct = O.moe_direct(x, topk, gates, w13f, w2f)
    e = rel_fro(f64_of(out), direct)
    say(f"tiny layer out vs fp32-weight direct rel fro {e:.3e}")
    assert e <= TOL


# ----------------------------------------------------------------------------
# full-size layer, sampled rows
# ----------------------------------------------------------------------------

def _full_layer(cfg, B, training):
    topk, gates, lam = W.routing_for(cfg)
    d = dims_of(cfg, B=B, training=training)
    plan, dest, _ = assert_plan_parity(d, topk, training=training)
    say("full layer maxvio", cfg.maxvio, "B", B, "replicas", len(plan.entries),
        "fallback", sum(1 for e in plan.entries if e.w < cfg.E))
    w13, w2 = W.expert_weights_torch(cfg.E, cfg.H, cfg.I, cfg.seed, DEV)
    xb = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    layer = MoonEPLayer(d, w13=w13, w2=w2, training=training)
    return topk, gates, xb, plan, dest, layer


def _expert_np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("B", [4, 3])
def test_full_layer_forward_sampled(B):
    cfg = W.CONFIGS["layer"]
    topk, gates, xb, plan, dest, layer = _full_layer(cfg, B, False)
    layer.forward(bf16_from_bits(xb), i32(topk), f32(gates))
    torch.cuda.synchronize()
    grp = O.groups(plan)
    rng = np.random.default_rng(1)
    kinds = {"home": [g for g in grp if g[4] == "home"], "slot": [g for g in grp if g[4] == "slot"],
             "fallback": [g for g in grp if g[4] == "fallback"]}
    picks = []
    for kind, lst in kinds.items():
        for gi in rng.permutation(len(lst))[:2]:
            picks.append(lst[gi])
    src_tok = np.empty(cfg.R * cfg.C, dtype=np.int64)
    src_tok[dest.ravel()] = np.repeat(np.arange(cfg.R * cfg.S), cfg.K)
    for (q, w, row0, rows, kind, idx) in picks:
        e = w if w < cfg.E else next(en.e for en in plan.entries if en.q == q and en.w == w)
        W13, W2 = _expert_np(layer.w13[e]), _expert_np(layer.w2[e])
        sel = row0 + rng.choice(rows, size=min(rows, 8), replace=False)
        assert np.array_equal(bits_of(layer.recv[torch.as_tensor(sel, device=DEV)]),
                              xb.reshape(-1, cfg.H)[src_tok[sel]])
        _, _, yref = O.swiglu_ffn(xb.reshape(-1, cfg.H)[src_tok[sel]], W13, W2)
        got = f64_of(layer.y[torch.as_tensor(sel, device=DEV)])
        err = max_row_rel(got, yref)
        say(f"  {kind} group q={q} w={w} e={e} rows={rows}: y max row rel {err:.3e}")
        assert err <= TOL


def test_full_layer_backward_experts():
    """Training at maxvio 8 with B=4: full dW of a fallback expert, a slot-replicated expert
    and a plain expert after reduce_grad, against the plan-free gradient; and the output and
    input gradient of sampled tokens (the unit-weight combine of the timed backward)."""
    cfg = W.CONFIGS["train"].with_(maxvio=8.0)
    topk, gates, xb, plan, dest, layer = _full_layer(cfg, cfg.B, True)
    doutb = W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    out = layer.forward(bf16_from_bits(xb), i32(topk), f32(gates)).clone()
    dx = layer.backward(bf16_from_bits(doutb), f32(gates))
    torch.cuda.synchronize()
    fb = sorted({en.e for en in plan.entries if en.w < cfg.E})
    sl = sorted({en.e for en in plan.entries if en.w >= cfg.E} - set(fb))
    rep = {en.e for en in plan.entries}
    plain = [e for e in range(cfg.E) if e not in rep and plan.L[e] > 0]
    chosen = ([fb[0]] if fb else []) + [sl[0], min(plain, key=lambda e: plan.L[e])]
    say("  experts", chosen, "fallback experts", fb)
    for e in chosen:
        W13 = layer.w13[e].cpu().view(torch.int16).numpy().view(np.uint16)
        W2 = layer.w2[e].cpu().view(torch.int16).numpy().view(np.uint16)
        # every (token, k) routed to e, whatever rank serves it
        ref13, ref2, _ = O.expert_grad_direct(xb, topk, gates, doutb, e, W13, W2)
        e13 = rel_fro(f64_of(layer.dw13[e]), ref13)
        e2 = rel_fro(f64_of(layer.dw2[e]), ref2)
        say(f"  expert {e} (L={plan.L[e]}): dW13 {e13:.3e} dW2 {e2:.3e}")
        assert e13 <= TOL and e2 <= TOL
    assert not layer.dw13_red.any() and not layer.dw2_red.any()
    # sampled tokens: out and dx rows (each sums K expert rows of y / drecv at full H)
    rng = np.random.default_rng(4)
    toks = [(int(r), int(s)) for r, s in zip(rng.integers(0, cfg.R, 4), rng.integers(0, cfg.S, 4))]
    cache = {}

    def weights_of(e):
        if e not in cache:
            cache[e] = (layer.w13[e].cpu().view(torch.int16).numpy().view(np.uint16),
                        layer.w2[e].cpu().view(torch.int16).numpy().view(np.uint16))
        return cache[e]

    ref_out, ref_dx = O.token_grad_direct(xb, topk, gates, doutb, toks, weights_of)
    idx_r = torch.as_tensor([r for r, _ in toks], device=DEV)
    idx_s = torch.as_tensor([s for _, s in toks], device=DEV)
    eo = max_row_rel(f64_of(out[idx_r, idx_s]), ref_out)
    ed = max_row_rel(f64_of(dx[idx_r, idx_s]), ref_dx)
    say(f"  sampled tokens: out max row rel {eo:.3e}, dx max row rel {ed:.3e}")
    assert eo <= TOL and ed <= TOL


def test_layer_stack_with_shared_pool():
    """Three layers sharing one prefetch pool [AT, TL;DR; TD, memory contract]: the output, the
    input gradient and every layer's weight gradients match the plan-free definition chained
    through the three layers; they are bit-identical to three layers with their own slots (each
    pooled layer prefetches again before its backward); and the pooled stack allocates two pools'
    worth less memory."""
    cfg = MID.with_(B=2)
    layers_n = 3
    topk, gates, _ = W.routing_for(cfg)
    tk, g = i32(topk), f32(gates)
    xb = bf16_from_bits(W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16"))
    dout = bf16_from_bits(W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16"))
    ws = []
    for l in range(layers_n):
        w13f, w2f = W.expert_weights_np(cfg.E, cfg.H, cfg.I, cfg.seed + 10 + l)
        ws.append((bf16_from_bits(W.bf16_bits(w13f)), bf16_from_bits(W.bf16_bits(w2f))))
    d = M.Dims.make(cfg.R, cfg.E, cfg.B, cfg.S, cfg.K, cfg.H, cfg.I, training=True)

    def run(pool):
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        if pool:
            p = MoonEPPool(cfg.R, cfg.B, cfg.H, cfg.I, training=True, device=DEV)
        stack = [MoonEPLayer(d, w13=a, w2=b, training=True, pool=p if pool else None) for a, b in ws]
        torch.cuda.synchronize()
        used = torch.cuda.memory_allocated() - before
        h = xb
        for L in stack:                     # forward through the stack (router output reused)
            h = L.forward(h, tk, g).clone()
        dh = dout
        for L in reversed(stack):           # backward in reverse layer order
            dh = L.backward(dh, g).clone()
        torch.cuda.synchronize()
        res = [h, dh] + [t.clone() for L in stack for t in (L.dw13, L.dw2)]
        return res, used

    ref, used_own = run(False)
    got, used_pool = run(True)
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))
    # the pooled stack against the plan-free definition chained layer by layer (each layer's
    # output and input gradient rounded to bf16, the type the layers hand on)
    wbits = [(W.bf16_bits(a), W.bf16_bits(b)) for a, b in
             (W.expert_weights_np(cfg.E, cfg.H, cfg.I, cfg.seed + 10 + l) for l in range(layers_n))]
    hs = [W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")]
    for (a, b) in wbits:
        hs.append(W.bf16_bits(O.moe_direct(hs[-1], topk, gates, a, b).astype(np.float32)))
    dh = W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    grads = [None] * layers_n
    for l in reversed(range(layers_n)):
        dxl, g13, g2 = O.moe_direct_backward(hs[l], topk, gates, wbits[l][0], wbits[l][1], dh)
        grads[l] = (g13, g2)
        dh = W.bf16_bits(dxl.astype(np.float32))
    e_out = rel_fro(f64_of(got[0]), W.bf16_to_f32(hs[-1]).astype(np.float64))
    e_dx = rel_fro(f64_of(got[1]), W.bf16_to_f32(dh).astype(np.float64))
    say(f"  pooled stack vs chained oracle: out {e_out:.3e}, dx {e_dx:.3e}")
    assert e_out <= TOL and e_dx <= TOL
    for l in range(layers_n):
        e13 = rel_fro(f64_of(got[2 + 2 * l]), grads[l][0])
        e2 = rel_fro(f64_of(got[3 + 2 * l]), grads[l][1])
        say(f"  layer {l}: dW13 {e13:.3e} dW2 {e2:.3e}")
        assert e13 <= TOL and e2 <= TOL
    saved = used_own - used_pool
    expect = (layers_n - 1) * MoonEPPool.nbytes(cfg.R, cfg.B, cfg.H, cfg.I, training=True)["total"]
    say(f"  pooled stack saves {saved / 2**20:.1f} MiB (expected {expect / 2**20:.1f} MiB)")
    assert abs(saved - expect) <= 2 * 2**20
