"""Oracle: exact minimum number of redundant experts and of migrated rows, to pin the plan rules.

TEST INFRASTRUCTURE ONLY.  Page abbreviations as in ``oracle.plan``.

The pages state that only a small number of duplicates is planned [AL, How it
works; TC, What we measured, Table 1 "copy slots"] and that a rank's duplicates
come from at most one other rank's home group [TC, Installation and
integration].  Two independent exact solvers give the least number of
(expert, serving rank) duplicates that balances every rank at C = S*K rows:

* ``min_replicas_enum``: brute force.  Candidate duplicate sets are enumerated
  in increasing size; each is tested with a max-flow transshipment (a library
  routine).  Network: source -> out_r (cap max(0, X_r)); out_h(e) -> expert e
  (cap L[e]); expert e -> in_q for each chosen (e, q); in_r -> sink (cap
  max(0, -X_r)); in_r -> out_r uncapped (a rank that receives rows may ship
  more of its own).  The set is feasible iff the flow saturates sum max(0, X).
* ``min_replicas_milp``: the same problem as a mixed-integer program (HiGHS via
  scipy), usable at sizes where enumeration is too slow.

The fewest rows that must leave their home rank ("migrated tokens" [TC, What we measured,
Table 1]) under the same one-remote-group property, two ways:

* ``min_migration_enum``: every map of ranks to the one remote home group they may serve (or
  none) is enumerated (tiny inputs); for each, the least rows moved is a linear program (a
  transshipment over the arcs the map allows, whose optimum is integral), solved with HiGHS.
* ``min_migration_milp``: one mixed-integer program over the arcs and the host choice.
Without the property the least is sum over ranks of max(0, X), every donor shipping its excess
straight to receivers (``one_group=False``).
"""
from __future__ import annotations

import itertools
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np
from scipy.optimize import Bounds, LinearConstraint, linprog, milp
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import maximum_flow


def _excess(L: Sequence[int], R: int, E: int, C: int) -> np.ndarray:
    G = E // R
    L = np.asarray(L, dtype=np.int64)
    return np.array([int(L[q * G:(q + 1) * G].sum()) - C for q in range(R)], dtype=np.int64)


def plan_is_feasible_flow(L: Sequence[int], R: int, E: int, C: int,
                          arcs: Iterable[Tuple[int, int]]) -> bool:
    """Can duplicates on exactly these (expert, rank) arcs balance every rank at C rows?"""
    G = E // R
    X = _excess(L, R, E, C)
    need = int(np.maximum(X, 0).sum())
    if need == 0:
        return True
    src, snk = 0, 1
    out_ = lambda r: 2 + r
    in_ = lambda r: 2 + R + r
    ex = lambda e: 2 + 2 * R + e
    nn = 2 + 2 * R + E
    big = int(np.sum(L)) + 1
    cap = {}

    def add(u, v, c):
        cap[(u, v)] = cap.get((u, v), 0) + int(c)

    for r in range(R):
        if X[r] > 0:
            add(src, out_(r), X[r])
        if X[r] < 0:
            add(in_(r), snk, -X[r])
        add(in_(r), out_(r), big)
    for e in range(E):
        if L[e] > 0:
            add(out_(e // G), ex(e), L[e])
    for (e, q) in arcs:
        add(ex(e), in_(q), L[e])
    rows, cols = zip(*cap.keys())
    m = csr_matrix((np.fromiter(cap.values(), dtype=np.int32), (rows, cols)), shape=(nn, nn))
    return int(maximum_flow(m, src, snk).flow_value) == need


def _one_group(arcs, G) -> bool:
    host = {}
    for (e, q) in arcs:
        d = e // G
        if host.setdefault(q, d) != d:
            return False
    return True


def min_replicas_enum(L: Sequence[int], R: int, E: int, C: int, one_group: bool = True,
                      max_size: Optional[int] = None) -> int:
    """Least duplicate count by exhaustive search (tiny inputs only: E*(R-1) candidate arcs)."""
    G = E // R
    L = np.asarray(L, dtype=np.int64)
    X = _excess(L, R, E, C)
    if not np.any(X):
        return 0
    donors = [d for d in range(R) if X[d] > 0]
    # a duplicate of an expert with no rows, or onto a rank that can never need one, never helps;
    # every candidate arc still has h(e) != q.
    cand = [(e, q) for e in range(E) for q in range(R) if e // G != q and L[e] > 0]
    limit = max_size if max_size is not None else len(cand)
    for size in range(1, limit + 1):
        for arcs in itertools.combinations(cand, size):
            if one_group and not _one_group(arcs, G):
                continue
            srcs = {e // G for (e, q) in arcs}
            if not set(donors) <= srcs:
                continue             # every donor must ship something
            if plan_is_feasible_flow(L, R, E, C, arcs):
                return size
    raise RuntimeError("no feasible duplicate set within the size limit")


def min_replicas_milp(L: Sequence[int], R: int, E: int, C: int, one_group: bool = True) -> int:
    """Least duplicate count as a MILP.

    Variables: z[e,q] in {0,1} (duplicate of e on rank q, h(e) != q), f[e,q] >= 0 rows it
    serves, y[q,d] in {0,1} (rank q hosts group d) when ``one_group``.
    Constraints: f <= L[e] z;  sum_q f[e,q] <= L[e];  for every rank q:
    P[q] - (rows of q's experts served elsewhere) + (rows q serves for others) = C;
    z[e,q] <= y[q,h(e)];  sum_d y[q,d] <= 1.   Objective: minimise sum z.
    """
    G = E // R
    L = np.asarray(L, dtype=np.int64)
    X = _excess(L, R, E, C)
    if not np.any(X):
        return 0
    arcs = [(e, q) for e in range(E) for q in range(R) if e // G != q]
    na = len(arcs)
    hosts = [(q, d) for q in range(R) for d in range(R) if d != q] if one_group else []
    nh = len(hosts)
    nv = 2 * na + nh                         # z | f | y
    cobj = np.zeros(nv)
    cobj[:na] = 1.0
    integrality = np.zeros(nv)
    integrality[:na] = 1
    integrality[2 * na:] = 1
    ub = np.concatenate([np.ones(na), np.array([L[e] for (e, q) in arcs], float), np.ones(nh)])
    rows, lo, hi = [], [], []

    def row(coefs, l, h):
        v = np.zeros(nv)
        for i, c in coefs:
            v[i] += c
        rows.append(v)
        lo.append(l)
        hi.append(h)

    for i, (e, q) in enumerate(arcs):
        row([(na + i, 1.0), (i, -float(L[e]))], -np.inf, 0.0)            # f <= L z
    for e in range(E):
        row([(na + i, 1.0) for i, (ee, q) in enumerate(arcs) if ee == e], -np.inf, float(L[e]))
    for q in range(R):
        co = [(na + i, -1.0) for i, (e, t) in enumerate(arcs) if e // G == q]
        co += [(na + i, 1.0) for i, (e, t) in enumerate(arcs) if t == q]
        row(co, float(-X[q]), float(-X[q]))                              # net in = -X[q]
    if one_group:
        hidx = {h: 2 * na + k for k, h in enumerate(hosts)}
        for i, (e, q) in enumerate(arcs):
            row([(i, 1.0), (hidx[(q, e // G)], -1.0)], -np.inf, 0.0)
        for q in range(R):
            row([(hidx[(q, d)], 1.0) for d in range(R) if d != q], -np.inf, 1.0)
    res = milp(cobj, integrality=integrality, bounds=Bounds(np.zeros(nv), ub),
               constraints=LinearConstraint(np.array(rows), np.array(lo), np.array(hi)))
    if not res.success:
        raise RuntimeError("MILP failed: " + str(res.message))
    return int(round(res.fun))


def _migration_rows(L, R, E, C, allowed, one_group):
    """Constraint rows of the least-migration problem over arcs (e, q), h(e) != q, allowed(e, q)."""
    G = E // R
    X = _excess(L, R, E, C)
    arcs = [(e, q) for e in range(E) for q in range(R) if e // G != q and L[e] > 0 and allowed(e, q)]
    return G, X, arcs


def min_migration_enum(L: Sequence[int], R: int, E: int, C: int) -> int:
    """Least migrated rows with at most one remote home group per rank, by enumerating every
    host map and solving the transshipment LP each allows (tiny inputs only: R**R maps)."""
    L = np.asarray(L, dtype=np.int64)
    best = None
    for hosts in itertools.product(range(-1, R), repeat=R):
        if any(h == q for q, h in enumerate(hosts)):
            continue
        G, X, arcs = _migration_rows(L, R, E, C, lambda e, q: hosts[q] == e // (E // R), True)
        if not np.any(X):
            return 0
        if not arcs:
            continue
        na = len(arcs)
        a_eq = np.zeros((R, na))
        for i, (e, q) in enumerate(arcs):
            a_eq[e // G, i] -= 1.0          # rows leave the home rank of e
            a_eq[q, i] += 1.0               # and arrive at q
        a_ub = np.zeros((E, na))
        for i, (e, q) in enumerate(arcs):
            a_ub[e, i] = 1.0                # an expert cannot give more rows than it has
        res = linprog(np.ones(na), A_ub=a_ub, b_ub=L.astype(float), A_eq=a_eq, b_eq=(-X).astype(float),
                      bounds=[(0, None)] * na, method="highs")
        if res.status == 0:
            v = int(round(res.fun))
            best = v if best is None else min(best, v)
    if best is None:
        raise RuntimeError("no feasible host map")
    return best


def min_migration_milp(L: Sequence[int], R: int, E: int, C: int, one_group: bool = True) -> int:
    """Least migrated rows as a MILP.

    Variables: f[e,q] >= 0 rows of e served on rank q != h(e); y[q,d] in {0,1} (rank q serves
    home group d) when ``one_group``.  Constraints: sum_q f[e,q] <= L[e]; for every rank q,
    (rows of others' experts served on q) - (rows of q's experts served elsewhere) = -X[q];
    f[e,q] <= L[e] y[q,h(e)]; sum_d y[q,d] <= 1.  Objective: minimise sum f."""
    L = np.asarray(L, dtype=np.int64)
    G, X, arcs = _migration_rows(L, R, E, C, lambda e, q: True, one_group)
    if not np.any(X):
        return 0
    na = len(arcs)
    hosts = [(q, d) for q in range(R) for d in range(R) if d != q] if one_group else []
    nh = len(hosts)
    hidx = {h: na + k for k, h in enumerate(hosts)}
    nv = na + nh
    cobj = np.zeros(nv)
    cobj[:na] = 1.0
    integrality = np.zeros(nv)
    integrality[na:] = 1
    ub = np.concatenate([np.array([L[e] for (e, q) in arcs], float), np.ones(nh)])
    rows, lo, hi = [], [], []

    def row(coefs, l, h):
        v = np.zeros(nv)
        for i, c in coefs:
            v[i] += c
        rows.append(v)
        lo.append(l)
        hi.append(h)

    for e in range(E):
        co = [(i, 1.0) for i, (ee, q) in enumerate(arcs) if ee == e]
        if co:
            row(co, -np.inf, float(L[e]))
    for q in range(R):
        co = [(i, -1.0) for i, (e, t) in enumerate(arcs) if e // G == q]
        co += [(i, 1.0) for i, (e, t) in enumerate(arcs) if t == q]
        row(co, float(-X[q]), float(-X[q]))
    if one_group:
        for i, (e, q) in enumerate(arcs):
            row([(i, 1.0), (hidx[(q, e // G)], -float(L[e]))], -np.inf, 0.0)
        for q in range(R):
            row([(hidx[(q, d)], 1.0) for d in range(R) if d != q], -np.inf, 1.0)
    res = milp(cobj, integrality=integrality, bounds=Bounds(np.zeros(nv), ub),
               constraints=LinearConstraint(np.array(rows), np.array(lo), np.array(hi)))
    if not res.success:
        raise RuntimeError("MILP failed: " + str(res.message))
    return int(round(res.fun))
