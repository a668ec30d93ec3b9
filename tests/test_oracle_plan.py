"""Pins of the CPU oracle's counts, maxvio, plan and destination rows.

Each check ties the oracle to something other than itself: hand-worked examples
(tests/golden/plan_worked.json), closed forms, the properties the MoonEP pages
fix, special cases with a textbook answer, and two independent exact solvers
for the least number of duplicates.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workload as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _plan_props(topk, plan, dest):
    """Properties the pages fix, checked on a plan and its destination rows."""
    R, S, K = topk.shape
    E, B, G, C = plan.E, plan.B, plan.G, plan.C
    # exactly S*K rows per rank (capacity check)
    assert np.all(plan.cu[:, E + B] == C)
    assert np.all(np.diff(plan.cu, axis=1) >= 0)
    # dest is a permutation of [0, R*C)
    flat = np.sort(dest.ravel())
    assert np.array_equal(flat, np.arange(R * C))
    # each row lands in a group whose weight row holds its expert
    row_expert = np.full(R * C, -1)
    slot_expert = {(en.q, en.w): en.e for en in plan.entries}
    for q in range(R):
        for w in range(E + B):
            lo, hi = plan.cu[q, w], plan.cu[q, w + 1]
            if hi == lo:
                continue
            e = w if w < E else slot_expert[(q, w)]
            row_expert[q * C + lo:q * C + hi] = e
    assert np.array_equal(row_expert[dest], topk)
    # at most one remote home group per rank; slots <= B; distinct (e, q) replicas
    host = {}
    for en in plan.entries:
        assert en.e // G != en.q
        assert host.setdefault(en.q, en.e // G) == en.e // G
    assert len({(en.e, en.q) for en in plan.entries}) == len(plan.entries)
    for q in range(R):
        assert sum(1 for en in plan.entries if en.q == q and en.w >= E) <= B
    # fallback exactly for entries beyond the slots
    for en in plan.entries:
        assert (en.w >= E) == (en.j < B)
    # migration is at least the excess that must leave the donors
    migrated = sum(en.a for en in plan.entries)
    assert migrated >= int(np.maximum(plan.X, 0).sum())
    # inside a group, source (rank, token) order is increasing
    src = np.empty(R * C, dtype=np.int64)
    src[dest.ravel()] = np.repeat(np.arange(R * S), K)
    for q in range(R):
        for w in range(E + B):
            lo, hi = q * C + plan.cu[q, w], q * C + plan.cu[q, w + 1]
            assert np.all(np.diff(src[lo:hi]) > 0)


# ----------------------------------------------------------------------------
# hand-worked examples
# ----------------------------------------------------------------------------

def _gold_cases():
    with open(os.path.join(GOLD, "plan_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _gold_cases(), ids=lambda c: c["name"])
def test_worked_examples(case):
    topk = np.array(case["topk"], dtype=np.int32)
    plan = O.make_plan(topk, case["E"], case["B"], rule=case.get("rule", "chain"))
    assert [[en.e, en.q, en.a] for en in plan.entries] == case["entries"]
    assert plan.cu.tolist() == case["cu"]
    dest = O.destinations(topk, plan)
    assert dest.tolist() == case["dest"]
    if "stats" in case:
        assert O.stats_vector(plan).tolist() == case["stats"]
    _plan_props(topk, plan, dest)


# ----------------------------------------------------------------------------
# counts and maxvio
# ----------------------------------------------------------------------------

def test_counts_hand_example():
    topk = np.array([[[0, 1], [1, 2]], [[3, 0], [2, 1]]], dtype=np.int32)
    c, L = O.expert_counts(topk, 4)
    assert c.tolist() == [[1, 2, 1, 0], [1, 1, 1, 1]]
    assert L.tolist() == [2, 3, 2, 1]


def test_maxvio_closed_forms():
    assert O.maxvio(np.full(16, 7)) == 0.0
    # all load on one of E experts: (a - a/E) / (a/E) = E - 1
    for E in (2, 16, 256):
        L = np.zeros(E)
        L[3 % E] = 1000
        assert O.maxvio(L) == pytest.approx(E - 1)
    # [2,1,1,0]: mean 1, max 2 -> 1
    assert O.maxvio([2, 1, 1, 0]) == pytest.approx(1.0)


def test_routing_validation():
    ok = np.array([[[0, 1]]], dtype=np.int32)
    O.validate_routing(ok, 4)
    with pytest.raises(O.RoutingError):
        O.make_plan(np.array([[[0, 4]]], dtype=np.int32), 4, 1)
    with pytest.raises(O.RoutingError):
        O.make_plan(np.array([[[2, 2]]], dtype=np.int32), 4, 1)
    with pytest.raises(O.RoutingError):
        O.make_plan(np.array([[[-1, 2]]], dtype=np.int32), 4, 1)


# ----------------------------------------------------------------------------
# special cases with closed forms
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("R,E,S,K", [(4, 16, 16, 2), (8, 64, 8, 4), (2, 8, 32, 1)])
def test_already_balanced_is_a_stable_sort(R, E, S, K):
    """All X[q] = 0: no duplicates; dest is the stable sort of pairs by (home rank, expert, r, s)."""
    G = E // R
    rng = np.random.default_rng(7)
    # every rank routes all its picks to its own home group -> P[q] = C for every q
    topk = np.empty((R, S, K), dtype=np.int32)
    for r in range(R):
        for s in range(S):
            topk[r, s] = r * G + rng.choice(G, size=K, replace=False)
    plan = O.make_plan(topk, E, 4)
    assert plan.entries == []
    dest = O.destinations(topk, plan)
    flat = topk.reshape(-1)
    order = np.argsort(flat, kind="stable")       # pairs by expert, then (r, s, k) order
    expect = np.empty_like(order)
    expect[order] = np.arange(flat.size)
    assert np.array_equal(dest.reshape(-1), expect)
    _plan_props(topk, plan, dest)


@pytest.mark.parametrize("rule", O.RULES)
@pytest.mark.parametrize("R,K,S", [(8, 8, 16), (8, 4, 16), (8, 2, 8), (4, 2, 32), (4, 4, 8)])
def test_single_hot_routing(R, K, S, rule):
    """Every token picks experts 0..K-1 (K <= G, K | R).

    L[e] = R*S = (R/K)*C for e < K, all in rank 0's group: rank 0 is the only donor with
    X = (R-1)*C and ranks 1..R-1 each need exactly C.  Best fit keeps reusing the lowest
    expert that still covers C, so receiver q is served by expert (q-1)*K//R; R-1 replicas,
    keep[K-1] = C, every other keep 0.
    """
    G = 8
    E = G * R
    topk = np.tile(np.arange(K, dtype=np.int32), (R, S, 1))
    plan = O.make_plan(topk, E, B=G, rule=rule)
    C = S * K
    assert len(plan.entries) == R - 1
    assert [(en.e, en.q, en.a) for en in plan.entries] == [((q - 1) * K // R, q, C) for q in range(1, R)]
    keep = np.zeros(E, dtype=np.int64)
    keep[K - 1] = C
    assert np.array_equal(plan.keep, keep)
    dest = O.destinations(topk, plan)
    _plan_props(topk, plan, dest)


@pytest.mark.parametrize("rule", O.RULES)
def test_slots_equal_group_never_fall_back(rule):
    """B = E/R covers every duplicate a rank can receive (one remote group of E/R experts)."""
    for seed in range(20):
        cfg = W.CONFIGS["tiny"].with_(seed=seed, lam=2.0)
        topk, _, _ = W.routing_for(cfg)
        plan = O.make_plan(topk, cfg.E, cfg.G, rule=rule)
        assert all(en.w >= cfg.E for en in plan.entries)


def test_fallback_does_not_change_rows_per_rank():
    """Fewer slots than duplicates: same replicas, some read the home row, still S*K per rank."""
    cfg = W.CONFIGS["tiny"].with_(lam=2.0)
    topk, _, _ = W.routing_for(cfg)
    full = O.make_plan(topk, cfg.E, cfg.G)
    for B in range(0, cfg.G + 1):
        p = O.make_plan(topk, cfg.E, B)
        assert [(e.e, e.q, e.a) for e in p.entries] == [(e.e, e.q, e.a) for e in full.entries]
        n_fb = sum(1 for en in p.entries if en.w < cfg.E)
        per_rank = np.bincount([en.q for en in p.entries], minlength=cfg.R)
        assert n_fb == int(np.maximum(per_rank - B, 0).sum())
        _plan_props(topk, p, O.destinations(topk, p))


# ----------------------------------------------------------------------------
# properties over configurations and seeds
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("rule", O.RULES)
@pytest.mark.parametrize("lam", [0.0, 0.25, 0.5, 1.0, 2.0])
def test_properties_seed_sweep_tiny(lam, rule):
    for seed in range(20):
        cfg = W.CONFIGS["tiny"].with_(seed=seed, lam=lam)
        topk, _, _ = W.routing_for(cfg)
        for B in (0, 2, cfg.B):
            plan = O.make_plan(topk, cfg.E, B, rule=rule)
            _plan_props(topk, plan, O.destinations(topk, plan))


@pytest.mark.parametrize("R,E,S,K,B,lam", [
    (8, 64, 128, 4, 2, 0.5), (8, 64, 128, 4, 8, 1.5), (2, 16, 64, 8, 1, 1.0),
    (1, 8, 32, 2, 0, 1.0), (8, 256, 64, 8, 4, 0.3), (4, 8, 64, 8, 2, 0.0),
])
@pytest.mark.parametrize("rule", O.RULES)
def test_properties_mid_shapes(R, E, S, K, B, lam, rule):
    cfg = W.Config("m", R=R, E=E, B=B, S=S, K=K, H=8, I=0, dtype="f32", lam=lam, seed=3)
    topk, _, _ = W.routing_for(cfg)
    plan = O.make_plan(topk, E, B, rule=rule)
    _plan_props(topk, plan, O.destinations(topk, plan))


@pytest.mark.slow
@pytest.mark.parametrize("rule", O.RULES)
@pytest.mark.parametrize("maxvio", [0.0, 0.5, 2.0, 4.0, 8.0])
def test_properties_full_size(maxvio, rule):
    cfg = W.CONFIGS["skew"].with_(maxvio=maxvio)
    topk, _, _ = W.routing_for(cfg)
    plan = O.make_plan(topk, cfg.E, cfg.B, rule=rule)
    dest = O.destinations(topk, plan)
    _plan_props(topk, plan, dest)
    if maxvio:
        assert abs(O.maxvio(plan.L) - maxvio) <= 0.01 * maxvio


# ----------------------------------------------------------------------------
# least number of duplicates
# ----------------------------------------------------------------------------

def test_milp_agrees_with_brute_force():
    """The MILP solver is pinned to exhaustive enumeration + max-flow on very small inputs."""
    checked = 0
    for (R, E, S, K) in [(3, 6, 8, 2), (4, 8, 8, 2)]:
        for lam in (0.5, 1.0, 2.0):
            for seed in range(4):
                cfg = W.Config("b", R=R, E=E, B=2, S=S, K=K, H=8, I=0, dtype="f32", lam=lam, seed=seed)
                topk, _, _ = W.routing_for(cfg)
                _, L = O.expert_counts(topk, E)
                m_enum = O.min_replicas_enum(L, R, E, S * K)
                assert O.min_replicas_milp(L, R, E, S * K) == m_enum
                assert O.min_replicas_milp(L, R, E, S * K, one_group=False) <= m_enum
                checked += 1
    assert checked == 24


def test_flow_check_on_a_plan():
    """The rule's own duplicate set is feasible by max-flow; dropping any one arc is not
    (each arc carries rows that no other arc can)."""
    cfg = W.CONFIGS["tiny"]
    topk, _, _ = W.routing_for(cfg)
    plan = O.make_plan(topk, cfg.E, cfg.B)
    arcs = [(en.e, en.q) for en in plan.entries]
    assert O.plan_is_feasible_flow(plan.L, cfg.R, cfg.E, cfg.C, arcs)
    assert not O.plan_is_feasible_flow(plan.L, cfg.R, cfg.E, cfg.C, arcs[:-1])


@pytest.mark.parametrize("lam", [0.0, 0.25, 0.5, 1.0, 2.0])
def test_rule_reaches_minimum_replicas(lam):
    """Tiny layer (R4 E16 S64 K2), seeds 0..99: both rules' duplicate count equals the least
    count any plan with at most one remote home group per rank can achieve."""
    for seed in range(100):
        cfg = W.CONFIGS["tiny"].with_(seed=seed, lam=lam)
        topk, _, _ = W.routing_for(cfg)
        least = None
        for rule in O.RULES:
            plan = O.make_plan(topk, cfg.E, cfg.B, rule=rule)
            least = least or O.min_replicas_milp(plan.L, cfg.R, cfg.E, cfg.C)
            assert len(plan.entries) == least, (lam, seed, rule)


# ----------------------------------------------------------------------------
# least number of migrated rows
# ----------------------------------------------------------------------------

def test_min_migration_milp_agrees_with_enumeration():
    """The least-migration MILP is pinned to enumeration of every host map with one LP each on
    very small inputs; without the one-group property it is the closed form sum max(0, X)."""
    checked = 0
    for (R, E, S, K) in [(3, 6, 8, 2), (4, 8, 8, 2)]:
        for lam in (0.5, 1.0, 2.0):
            for seed in range(3):
                cfg = W.Config("b", R=R, E=E, B=2, S=S, K=K, H=8, I=0, dtype="f32", lam=lam, seed=seed)
                topk, _, _ = W.routing_for(cfg)
                _, L = O.expert_counts(topk, E)
                G = E // R
                X = np.array([L[q * G:(q + 1) * G].sum() for q in range(R)]) - S * K
                assert O.min_migration_milp(L, R, E, S * K) == O.min_migration_enum(L, R, E, S * K)
                assert O.min_migration_milp(L, R, E, S * K, one_group=False) == int(np.maximum(X, 0).sum())
                checked += 1
    assert checked == 18


@pytest.mark.slow
@pytest.mark.parametrize("workload", ["lognormal sigma 1", "lognormal sigma 5", "zipf maxvio 4",
                                      "zipf maxvio 8"])
def test_lowmig_reaches_least_migration(workload):
    """Under strong skew the low-migration rule moves exactly the least number of rows any plan
    with at most one remote home group per rank can (the exact MILP optimum), and fewer than the
    chain rule; both plans keep their properties."""
    kind, _, v = workload.split()
    if kind == "lognormal":
        c = W.LOGNORMAL
        topk = np.array(W.lognormal_routing(c["R"], c["S"], c["E"], c["K"], float(v))[0])
        R, E, C = c["R"], c["E"], c["S"] * c["K"]
    else:
        cfg = W.CONFIGS["skew"].with_(maxvio=float(v))
        topk, _, _ = W.routing_for(cfg)
        R, E, C = cfg.R, cfg.E, cfg.C
    lo = O.make_plan(topk, E, 4, rule="lowmig")
    ch = O.make_plan(topk, E, 4)
    _plan_props(topk, lo, O.destinations(topk, lo))
    mig_lo = sum(en.a for en in lo.entries)
    mig_ch = sum(en.a for en in ch.entries)
    assert mig_lo == O.min_migration_milp(lo.L, R, E, C)
    assert mig_lo < mig_ch


# ----------------------------------------------------------------------------
# memory contract arithmetic
# ----------------------------------------------------------------------------

def test_memory_table2():
    with open(os.path.join(GOLD, "memory_table2.json")) as f:
        g = json.load(f)
    sh = g["shape"]
    gib = 2.0 ** 30
    for row in g["rows"]:
        b = O.buffer_bytes(row["B"], sh["S"], sh["K"], sh["H"], sh["I"],
                           projections=sh["projections"], training=row["mode"] == "training")
        for k in ("prefetch", "reduce", "dispatch", "total"):
            assert abs(b[k] / gib - row[k + "_gib"]) <= 0.0051, (row["mode"], k)
    hb = O.buffer_bytes(0, sh["S"], sh["K"], sh["H"], sh["I"], E_home=32)["home_weights"] / gib
    assert abs(hb - g["home_weights_gib_per_rank_E_over_R_32"]) < 0.05


# ----------------------------------------------------------------------------
# lognormal expert popularity (thakicloud.com post, "What we measured", Table 1 setup)
# ----------------------------------------------------------------------------

def _table1():
    with open(os.path.join(os.path.dirname(__file__), "golden", "lognormal_table1.json")) as f:
        return json.load(f)


def test_lognormal_generator_is_a_popularity_sampler():
    """sigma = 0 routes uniformly (expert loads within a few standard deviations of the mean);
    K distinct experts per token; larger sigma concentrates load (rank peak/mean rises)."""
    c = W.LOGNORMAL
    peaks = []
    for sg in c["sigmas"]:
        topk, gates = W.lognormal_routing(c["R"], c["S"], c["E"], c["K"], sg)
        O.validate_routing(np.array(topk), c["E"])
        np.testing.assert_allclose(gates.sum(axis=-1), 1.0, atol=1e-5)
        L = np.bincount(np.asarray(topk).ravel(), minlength=c["E"])
        P = L.reshape(c["R"], -1).sum(axis=1)
        peaks.append(P.max() / (c["S"] * c["K"]))
        if sg == 0.0:
            mean = c["R"] * c["S"] * c["K"] / c["E"]
            assert np.abs(L - mean).max() <= 6 * np.sqrt(mean)
    assert all(a < b for a, b in zip(peaks, peaks[1:]))


@pytest.mark.parametrize("sigma", [0.0, 0.5, 1.0, 2.0, 5.0])
def test_lognormal_plan_properties(sigma):
    """Every rank gets exactly S*K rows at every skew; the copy count stays small (the post saw
    7-9 with its generator); migration is at least its lower bound."""
    c = W.LOGNORMAL
    topk, _ = W.lognormal_routing(c["R"], c["S"], c["E"], c["K"], sigma)
    topk = np.array(topk)
    plan = O.make_plan(topk, c["E"], 4)
    _plan_props(topk, plan, O.destinations(topk, plan))
    low = O.make_plan(topk, c["E"], 4, rule="lowmig")
    _plan_props(topk, low, O.destinations(topk, low))
    st = O.stats_vector(plan)
    P = np.bincount(topk.ravel(), minlength=c["E"]).reshape(c["R"], -1).sum(axis=1)
    assert st[8] == P.max() and st[9] == P.min()      # baseline (home-pinned) rank loads
    assert np.all(plan.cu[:, -1] == c["S"] * c["K"])  # after planning: exactly S*K everywhere
    assert st[5] >= st[6]
    assert 0 <= st[1] <= 12
    table = {row[0]: row for row in _table1()["rows"]}
    assert sigma in table     # the post's sweep points
