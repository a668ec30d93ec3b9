"""GPU parity of planning, dispatch and combine against the CPU oracle.

Plan, cu_seqlens, dest, stats and permuted rows must be bit-exact; combine within
1e-2 (max over tokens of the row-wise relative L2 error) of the float64 oracle.
"""
import json
import os

import numpy as np
import pytest
import torch

import balanced_token_dispatch_moonep_amd as M
import oracle as O
import workload as W

from gpu_util import (DEV, say, dims_of, i32, f32, bf16_from_bits, bits_of, f64_of, rows_tensor,
                      run_plan, assert_plan_parity, max_row_rel)

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "plan_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _gold(), ids=lambda c: c["name"])
def test_plan_worked_examples(case):
    say("plan worked example", case["name"])
    topk = np.array(case["topk"], dtype=np.int32)
    d = M.Dims.make(case["R"], case["E"], case["B"], case["S"], case["K"], 8, plan_rule=case.get("rule", "chain"))
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d, topk)
    assert dd.cpu().numpy().tolist() == case["dest"]
    assert cu.cpu().numpy().tolist() == case["cu"]


RULES = ("chain", "lowmig")


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("lam", [0.0, 0.5, 1.0, 2.0])
@pytest.mark.parametrize("B", [0, 2, 4])
def test_plan_tiny_sweep(lam, B, rule):
    for seed in range(5):
        cfg = W.CONFIGS["tiny"].with_(lam=lam, seed=seed)
        topk, _, _ = W.routing_for(cfg)
        say("plan tiny", lam, B, seed, rule)
        assert_plan_parity(dims_of(cfg, B=B, training=True, rule=rule), topk, training=True)


def _degenerate_routing(kind, R, E, S, K):
    G = E // R
    s_idx = np.arange(S)[None, :, None]
    r_idx = np.arange(R)[:, None, None]
    k_idx = np.arange(K)[None, None, :]
    if kind == "single_hot":        # every token picks experts 0..K-1 (all on rank 0)
        t = np.broadcast_to(k_idx, (R, S, K))
    elif kind == "own_home":        # every token stays in its own rank's home group: no replica
        t = r_idx * G + (s_idx * K + k_idx) % G
    elif kind == "round_robin":     # every expert gets exactly S*K*R/E pairs
        t = (r_idx * S * K + s_idx * K + k_idx) % E
    elif kind == "next_rank":       # every token picks the next rank's home group
        t = ((r_idx + 1) % R) * G + (s_idx * K + k_idx) % G
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(t, dtype=np.int32)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("kind", ["single_hot", "own_home", "round_robin", "next_rank"])
@pytest.mark.parametrize("B,training", [(0, False), (2, False), (4, True)])
def test_plan_degenerate_routings(kind, B, training, rule):
    """Routings at the ends of the method's range, bit-exact against the oracle: all load on one
    rank (most replicas, fallback when slots run out), none to move, and every pair remote."""
    R, E, S, K = 8, 64, 96, 4
    topk = _degenerate_routing(kind, R, E, S, K)
    say("plan degenerate", kind, B, training, rule)
    d = M.Dims.make(R, E, B, S, K, 8, training=training, plan_rule=rule)
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d, topk, training=training)
    if kind in ("own_home", "round_robin", "next_rank"):
        assert len(plan.entries) == 0          # every rank already serves exactly S*K rows
    if kind == "single_hot":
        assert len(plan.entries) >= R - 1      # rank 0 sheds (R-1)*S*K rows to the others


@pytest.mark.parametrize("R,E,S,K,B,lam", [
    (8, 64, 128, 4, 2, 0.5), (8, 64, 130, 4, 8, 1.5), (2, 16, 64, 8, 1, 1.0),
    (1, 8, 32, 2, 0, 1.0), (8, 256, 64, 8, 4, 0.3), (4, 8, 65, 8, 2, 0.0), (16, 512, 96, 8, 3, 0.8),
    (3, 12, 200, 3, 1, 1.2),
    # 64 home experts per rank, the most a rank's group may hold (one lane per expert in the
    # planner's replica chain)
    (2, 128, 128, 8, 4, 1.0), (8, 512, 96, 8, 4, 0.8), (4, 256, 64, 8, 0, 1.5),
    # 4,160 chunks (a ragged last one per rank): more than 512 histogram segments, so the
    # decision kernel's threads each read several segment status words and sum their experts'
    # segment totals in several batches
    (64, 128, 4150, 2, 2, 1.0),
])
@pytest.mark.parametrize("rule", RULES)
def test_plan_shapes(R, E, S, K, B, lam, rule):
    cfg = W.Config("m", R=R, E=E, B=B, S=S, K=K, H=8, I=0, dtype="f32", lam=lam, seed=3)
    topk, _, _ = W.routing_for(cfg)
    say("plan shape", R, E, S, K, B, lam, rule)
    assert_plan_parity(dims_of(cfg, rule=rule), topk)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("maxvio", [0.0, 0.5, 2.0, 4.0, 8.0])
def test_plan_full_size(maxvio, rule):
    cfg = W.CONFIGS["skew"].with_(maxvio=maxvio)
    topk, _, _ = W.routing_for(cfg)
    say("plan full size maxvio", maxvio, rule)
    for B in (4, 3):
        plan, dest, (ws, cu, dd, st) = assert_plan_parity(dims_of(cfg, B=B, rule=rule), topk)
        s = st.cpu().numpy()
        assert s[13] == cfg.R * cfg.C and s[0] == 0


def test_plan_is_deterministic():
    cfg = W.CONFIGS["skew"].with_(maxvio=8.0)
    topk, _, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    tk = i32(topk)
    first = [t.cpu().clone() for t in run_plan(d, topk, tk)[1:]]
    for _ in range(3):
        again = run_plan(d, topk, tk)[1:]
        for a, b in zip(first, again):
            assert torch.equal(a, b.cpu())


def test_plan_invalid_routing_sets_status_and_no_rows():
    cfg = W.CONFIGS["tiny"]
    topk, _, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    bad = topk.copy()
    bad[1, 3, 0] = cfg.E          # out of range
    _, cu, dest, st = run_plan(d, bad)
    assert st.cpu().numpy()[0] & M.ST_BAD_ID
    assert (dest.cpu().numpy() == -1).all()
    assert (cu.cpu().numpy() == 0).all()
    dup = topk.copy()
    dup[2, 5, 1] = dup[2, 5, 0]   # duplicate expert in one token
    _, cu, dest, st = run_plan(d, dup)
    assert st.cpu().numpy()[0] & M.ST_DUP_ID
    assert (dest.cpu().numpy() == -1).all()
    # dispatch and combine skip rows whose dest is -1
    x = torch.randn((cfg.R, cfg.S, cfg.H), device=DEV)
    recv = torch.full((cfg.R * cfg.C, cfg.H), 3.0, device=DEV)
    M.moonep_dispatch(d, dest, x, None, recv)
    out = torch.full_like(x, 5.0)
    M.moonep_combine(d, dest, recv, None, out)
    torch.cuda.synchronize()
    assert bool((recv == 3.0).all()) and bool((out == 0.0).all())


def test_plan_training_fallback_flag():
    cfg = W.CONFIGS["tiny"].with_(lam=2.0)
    topk, _, _ = W.routing_for(cfg)
    plan, _, (_, _, _, st) = assert_plan_parity(dims_of(cfg, B=0, training=True), topk, training=True)
    assert plan.entries and (st.cpu().numpy()[0] & M.ST_TRAIN_FALLBACK)


# ----------------------------------------------------------------------------
# dispatch
# ----------------------------------------------------------------------------

def _layer_inputs(cfg, B=None):
    topk, gates, _ = W.routing_for(cfg)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, cfg.dtype)
    d = dims_of(cfg, B=B)
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d, topk)
    return topk, gates, x, d, plan, dest, dd


@pytest.mark.parametrize("name,over", [
    ("tiny", {}), ("tiny", {"S": 100, "lam": 2.0}),
    ("balanced", {"S": 256, "H": 512}), ("skew", {"S": 192, "H": 1032, "maxvio": 8.0}),
])
def test_dispatch_bitexact(name, over):
    cfg = W.CONFIGS[name].with_(**over)
    topk, gates, x, d, plan, dest, dd = _layer_inputs(cfg)
    say("dispatch", name, over)
    xt = rows_tensor(x)
    canary = float("nan")
    recv = torch.full((cfg.R * cfg.C, cfg.H), canary, dtype=xt.dtype, device=DEV)
    M.moonep_dispatch(d, dd, xt, None, recv)
    torch.cuda.synchronize()
    ref = O.dispatch(dest, x)
    got = recv.cpu().numpy() if cfg.dtype == "f32" else bits_of(recv)
    assert got.tobytes() == ref.tobytes()          # every row written, bit for bit


@pytest.mark.parametrize("maxvio", [0.0, 8.0])
def test_dispatch_full_size(maxvio):
    cfg = W.CONFIGS["skew"].with_(maxvio=maxvio)
    topk, _, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    plan = O.make_plan(topk, cfg.E, cfg.B)
    dest = O.destinations(topk, plan)
    say("dispatch full size maxvio", maxvio)
    _, cu, dd, st = run_plan(d, topk)
    np.testing.assert_array_equal(dd.cpu().numpy(), dest)
    x = bf16_from_bits(W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16"))
    recv = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.bfloat16, device=DEV)
    recv.view(torch.int16).fill_(-1)
    M.moonep_dispatch(d, dd, x, None, recv)
    torch.cuda.synchronize()
    # dest is a permutation (checked against the oracle above): each row must equal its token
    src_tok = torch.empty(cfg.R * cfg.C, dtype=torch.long, device=DEV)
    src_tok[dd.view(-1).long()] = torch.arange(cfg.R * cfg.S, device=DEV).repeat_interleave(cfg.K)
    xs = x.view(-1, cfg.H)
    for lo in range(0, cfg.R * cfg.C, 32768):
        hi = lo + 32768
        assert torch.equal(recv[lo:hi].view(torch.int16), xs[src_tok[lo:hi]].view(torch.int16))


@pytest.mark.parametrize("name,over", [
    ("skew", {"S": 128, "H": 512, "maxvio": 4.0}),      # K = 8: scales loaded before the row
    ("balanced", {"S": 64, "H": 264, "K": 3}),          # K read at run time, ragged last batch
    ("tiny", {}),                                       # float32 rows
    # K = 8 and rows that are whole batches of 128 vectors: the unchecked full-row form that the
    # benchmark's combine backward runs at H = 7168 (one batch at H = 1024, two at 2048)
    ("skew", {"S": 96, "H": 1024, "maxvio": 4.0}),
    ("skew", {"S": 64, "H": 2048, "maxvio": 8.0}),
])
def test_dispatch_row_scale(name, over):
    cfg = W.CONFIGS[name].with_(**over)
    topk, gates, x, d, plan, dest, dd = _layer_inputs(cfg)
    say("dispatch row scale", name, over)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, 1, cfg.dtype)
    recv = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16,
                       device=DEV)
    M.moonep_dispatch(d, dd, rows_tensor(dout), f32(gates), recv)
    torch.cuda.synchronize()
    ref = O.dispatch(dest, dout, row_scale=gates)
    got = f64_of(recv)
    # one float32 product rounded once to the row type: within half an ulp of it
    # (bf16: 2^-9 relative, float32: 2^-24 relative)
    tol = 2.0 ** -23 if cfg.dtype == "f32" else 2.0 ** -8
    assert np.all(np.abs(got - ref) <= np.abs(ref) * tol + 1e-30)


def test_dispatch_row_scale_full_size_sampled():
    """The combine backward exactly as the benchmark runs it (H = 7168, K = 8, full-row form):
    every row of 64 sampled tokens against the oracle's scaled dispatch of those tokens."""
    cfg = W.CONFIGS["skew"].with_(maxvio=4.0)
    topk, gates, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    say("dispatch row scale full size (sampled)")
    _, cu, dd, st = run_plan(d, topk)
    plan = O.make_plan(topk, cfg.E, cfg.B)
    dest = O.destinations(topk, plan)
    np.testing.assert_array_equal(dd.cpu().numpy(), dest)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    dy = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.bfloat16, device=DEV)
    M.moonep_dispatch(d, dd, bf16_from_bits(dout), f32(gates), dy)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    toks = [(int(r), int(s)) for r, s in zip(rng.integers(0, cfg.R, 64), rng.integers(0, cfg.S, 64))]
    # the sampled tokens as a one-rank problem whose rows land in arrival order
    sub_dest = np.arange(len(toks) * cfg.K).reshape(1, len(toks), cfg.K)
    sub_x = np.stack([dout[r, s] for r, s in toks])[None]
    sub_g = np.stack([gates[r, s] for r, s in toks])[None]
    ref = O.dispatch(sub_dest, sub_x, row_scale=sub_g)
    rows = torch.as_tensor(np.array([dest[r, s, k] for r, s in toks for k in range(cfg.K)]), device=DEV)
    got = f64_of(dy[rows])
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,over,gated", [
    ("tiny", {}, True), ("tiny", {"S": 100, "lam": 2.0}, False),
    ("skew", {"S": 192, "H": 1032, "maxvio": 8.0}, True), ("balanced", {"S": 128, "H": 512, "K": 3}, True),
    ("balanced", {"S": 64, "H": 256, "K": 5}, False),
    # rows of several 7 KiB chunks (K = 8): both forms the benchmark runs at H = 7168 (unit
    # weights, bounds-checked; gated, full-row) and a partial last chunk at H = 4096
    ("skew", {"S": 64, "H": 4096, "maxvio": 4.0}, False), ("skew", {"S": 64, "H": 7168, "maxvio": 4.0}, False),
    ("skew", {"S": 64, "H": 7168, "maxvio": 4.0}, True),
])
def test_combine_vs_oracle(name, over, gated):
    cfg = W.CONFIGS[name].with_(**over)
    topk, gates, x, d, plan, dest, dd = _layer_inputs(cfg)
    say("combine", name, over, gated)
    rng = np.random.default_rng(11)
    yv = rng.standard_normal((cfg.R * cfg.C, cfg.H)).astype(np.float32)
    y = yv if cfg.dtype == "f32" else W.bf16_bits(yv)
    out = torch.empty((cfg.R, cfg.S, cfg.H), dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16,
                      device=DEV)
    M.moonep_combine(d, dd, rows_tensor(y), f32(gates) if gated else None, out)
    torch.cuda.synchronize()
    ref = O.combine(dest, y, gates if gated else None)
    err = max_row_rel(f64_of(out), ref)
    say("  max row rel err", err)
    assert err <= 1e-2


@pytest.mark.parametrize("maxvio", [0.0, 4.0])
def test_round_trip_full_size(maxvio):
    """Identity experts: combine(dispatch(x)) with gates summing to 1 returns x (bf16 rounding)."""
    cfg = W.CONFIGS["skew"].with_(maxvio=maxvio)
    topk, gates, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    say("round trip full size", maxvio)
    _, cu, dd, st = run_plan(d, topk)
    xb = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    x = bf16_from_bits(xb)
    recv = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x)
    M.moonep_dispatch(d, dd, x, None, recv)
    g = f32(gates)
    M.moonep_combine(d, dd, recv, g, out)
    torch.cuda.synchronize()
    num = (out.float() - x.float()).norm(dim=-1)
    den = x.float().norm(dim=-1)
    assert float((num / den).max()) <= 1e-2
    # sampled tokens against the oracle's combine
    plan = O.make_plan(topk, cfg.E, cfg.B)
    dest = O.destinations(topk, plan)
    np.testing.assert_array_equal(dd.cpu().numpy(), dest)
    rng = np.random.default_rng(5)
    for (r, s) in zip(rng.integers(0, cfg.R, 64), rng.integers(0, cfg.S, 64)):
        ref = sum(float(gates[r, s, k]) * W.bf16_to_f32(xb[r, s]).astype(np.float64) for k in range(cfg.K))
        got = f64_of(out[r, s])
        assert np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref)


# ----------------------------------------------------------------------------
# staged (non-zero-copy) baseline: same results as the fused calls
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,over,scaled", [
    ("tiny", {}, False), ("tiny", {"S": 100, "lam": 2.0}, True),
    ("skew", {"S": 192, "H": 1032, "maxvio": 8.0}, True), ("balanced", {"S": 128, "H": 512, "K": 3}, False),
])
def test_staged_matches_fused(name, over, scaled):
    cfg = W.CONFIGS[name].with_(**over)
    topk, gates, x, d, plan, dest, dd = _layer_inputs(cfg)
    say("staged", name, over, scaled)
    xt = rows_tensor(x)
    g = f32(gates)
    M_ = cfg.R * cfg.C
    recv = torch.empty((M_, cfg.H), dtype=xt.dtype, device=DEV)
    recv2 = torch.full_like(recv, float("nan"))
    stage = torch.full_like(recv, float("nan"))
    M.moonep_dispatch(d, dd, xt, g if scaled else None, recv)
    M.moonep_dispatch_staged(d, dd, xt, g if scaled else None, stage, recv2)
    torch.cuda.synchronize()
    asbits = (lambda t: t.cpu().numpy()) if cfg.dtype == "f32" else bits_of
    assert asbits(recv2).tobytes() == asbits(recv).tobytes()
    if not scaled:   # arrival order: row (r, s, k) holds token (r, s)
        ref = np.repeat(x.reshape(cfg.R * cfg.S, cfg.H), cfg.K, axis=0)
        assert asbits(stage).tobytes() == np.ascontiguousarray(ref).tobytes()
        assert asbits(recv2).tobytes() == O.dispatch(dest, x).tobytes()
    rng = np.random.default_rng(3)
    yv = rng.standard_normal((M_, cfg.H)).astype(np.float32)
    y = rows_tensor(yv if cfg.dtype == "f32" else W.bf16_bits(yv))
    out = torch.empty((cfg.R, cfg.S, cfg.H), dtype=xt.dtype, device=DEV)
    out2 = torch.full_like(out, float("nan"))
    M.moonep_combine(d, dd, y, g, out)
    M.moonep_combine_staged(d, dd, y, g, stage, out2)
    torch.cuda.synchronize()
    assert asbits(out2).tobytes() == asbits(out).tobytes()
    # the gather to arrival order: stage[p] = y[dest[p]]
    idx = torch.from_numpy(dest.reshape(-1).astype(np.int64)).to(DEV)
    assert torch.equal(stage.view(torch.int16) if cfg.dtype != "f32" else stage,
                       (y[idx].view(torch.int16) if cfg.dtype != "f32" else y[idx]))


def test_staged_full_size_matches_fused():
    cfg = W.CONFIGS["skew"].with_(maxvio=4.0)
    topk, gates, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    say("staged full size")
    _, cu, dd, st = run_plan(d, topk)
    x = bf16_from_bits(W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16"))
    g = f32(gates)
    recv = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.bfloat16, device=DEV)
    recv2 = torch.empty_like(recv)
    stage = torch.empty_like(recv)
    M.moonep_dispatch(d, dd, x, None, recv)
    M.moonep_dispatch_staged(d, dd, x, None, stage, recv2)
    out = torch.empty_like(x)
    out2 = torch.empty_like(x)
    M.moonep_combine(d, dd, recv, g, out)
    M.moonep_combine_staged(d, dd, recv2, g, stage, out2)
    torch.cuda.synchronize()
    assert torch.equal(recv.view(torch.int16), recv2.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("sigma", [0.0, 0.5, 1.0, 2.0, 5.0])
def test_plan_lognormal(sigma, rule):
    """The planner workload of the thakicloud.com post (Table 1 setup), bit-exact to the oracle."""
    c = W.LOGNORMAL
    topk, _ = W.lognormal_routing(c["R"], c["S"], c["E"], c["K"], sigma)
    d = M.Dims.make(c["R"], c["E"], 4, c["S"], c["K"], 128, plan_rule=rule)
    say("plan lognormal sigma", sigma, rule)
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d, np.array(topk))
    assert np.all(cu.cpu().numpy()[:, -1] == c["S"] * c["K"])


def test_plan_dispatch_combine_max_dims():
    """The largest dims the library accepts for the plan tables: 64 ranks, 1024 experts (16 per
    rank), 64 slots, top-16."""
    cfg = W.Config("max", R=64, E=1024, B=64, S=64, K=16, H=64, I=0, dtype="bf16", lam=1.0, seed=4)
    topk, gates, _ = W.routing_for(cfg)
    d = dims_of(cfg)
    say("max dims")
    plan, dest, (ws, cu, dd, st) = assert_plan_parity(d, topk)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "bf16")
    recv = torch.empty((cfg.R * cfg.C, cfg.H), dtype=torch.bfloat16, device=DEV)
    M.moonep_dispatch(d, dd, bf16_from_bits(x), None, recv)
    out = torch.empty((cfg.R, cfg.S, cfg.H), dtype=torch.bfloat16, device=DEV)
    M.moonep_combine(d, dd, recv, f32(gates), out)
    torch.cuda.synchronize()
    assert bits_of(recv).tobytes() == O.dispatch(dest, x).tobytes()
    assert max_row_rel(f64_of(out), O.combine(dest, O.dispatch(dest, x), gates)) <= 1e-2


def test_binding_rejects_wrong_workspace():
    """Every entry point that reads the plan workspace checks its size before any launch."""
    say("binding: workspace size checks")
    d = M.Dims.make(R=2, E=4, B=1, S=64, K=2, H=64, I=64, training=True)
    n = M.moonep_plan_workspace_bytes(d)
    for size in (n - 256, n + 256):
        bad = torch.zeros(size, dtype=torch.uint8, device=DEV)
        topk = torch.zeros((d.R, d.S, d.K), dtype=torch.int32, device=DEV)
        for call in (lambda: M.moonep_plan(d, topk, bad, None, None, None),
                     lambda: M.moonep_prefetch(d, bad, None, None, None, None),
                     lambda: M.moonep_grouped_ffn(d, bad, *[None] * 9),
                     lambda: M.moonep_grouped_ffn_backward(d, bad, *[None] * 14),
                     lambda: M.moonep_reduce_grad(d, bad, None, None, None, None)):
            with pytest.raises(ValueError, match="plan_ws"):
                call()
