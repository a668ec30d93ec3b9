"""Oracle: expert counts, maxvio, the redundant-expert plan and destination rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (title, site):
  [AT] "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert Parallelism
       Library for MoE Training", aitrending.vip
  [AL] "MoonshotAI/MoonEP", agentlenshq.com
  [TD] "MoonEP balances AI experts in MoE models ...", twodots.gr
  [TC] "The Busiest Rank Sets Your Step Time: Running MoonEP's Planning Code
       Ourselves", thakicloud.com

What the pages fix about the plan:
  * every rank ends up with exactly S*K (token, k) rows whatever the routing
    [TD, summary and FAQ; TC, Overview; AT, TL;DR];
  * the plan is made online from this step's router output (topk_experts /
    tokens_per_expert) by duplicating a small number of experts onto ranks with
    spare room [TC, "What the technique is" and its flowchart; AL, How it works];
  * a rank's duplicates come from at most one other rank's home experts, which
    is why training needs B = E/R slots [TC, Installation and integration];
  * weight rows [0, E) are the home experts (rank r owns rows r*E/R .. (r+1)*E/R-1),
    rows [E, E+B) are this rank's prefetch slots, and cu_seqlens (per weight row)
    selects the active rows of the grouped GEMM [TD, memory contract; TC,
    Installation and integration, weight-tensor flowchart];
  * with fewer slots than needed (inference B=3-4) the surplus duplicates read the
    home rank's row instead: slower, same result [TD, memory contract and FAQ;
    TC, Installation and integration];
  * the planner raises when a rank's allocation exceeds its capacity S*K
    [TC, What we measured, text under Table 1].

The pages give the properties, not the algorithm.  The rule implemented here
(the plainest one with all of them) is written out step by step in
``make_plan``; every tie is broken towards the lower rank or expert id.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

# status bits (device status word and oracle errors share this numbering)
ST_BAD_ID = 1          # an expert id outside [0, E)
ST_DUP_ID = 2          # a token lists the same expert twice
ST_CAPACITY = 4        # some rank does not end with exactly S*K rows
ST_OVERFLOW = 8        # more plan entries than the entry table holds
ST_TRAIN_FALLBACK = 16  # training with a fallback replica (B < E/R); informational

STAT_NAMES = (
    "status", "replicas", "slot_replicas", "fallback_replicas", "fallback_rows",
    "migrated_rows", "migration_bound", "max_expert_load", "max_rank_load",
    "min_rank_load", "donors", "receivers", "max_replicas_per_rank", "total_rows",
    "reserved14", "reserved15",
)


class RoutingError(ValueError):
    """Invalid router output (id out of range or duplicate expert in one token)."""


class CapacityError(RuntimeError):
    """A rank's planned row count differs from S*K (cannot happen for a valid plan)."""


def validate_routing(topk: np.ndarray, E: int) -> None:
    """Router outputs must name K distinct experts in [0, E) per token [TC, flowchart input]."""
    t = np.asarray(topk)
    if t.ndim != 3:
        raise RoutingError("topk must be [R, S, K]")
    if t.size and (t.min() < 0 or t.max() >= E):
        raise RoutingError("expert id outside [0, E)")
    st = np.sort(t, axis=2)
    if t.shape[2] > 1 and np.any(st[:, :, 1:] == st[:, :, :-1]):
        raise RoutingError("duplicate expert within one token's top-K")


def expert_counts(topk: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """c[r, e] = number of (s, k) on rank r routed to e; L[e] = sum_r c[r, e].

    tokens_per_expert of the router output [TC, "What the technique is" flowchart].
    """
    R = topk.shape[0]
    c = np.zeros((R, E), dtype=np.int64)
    for r in range(R):
        c[r] = np.bincount(np.asarray(topk[r]).ravel(), minlength=E)
    return c, c.sum(axis=0)


def maxvio(L: np.ndarray) -> float:
    """Imbalance metric: (max load - mean load) / mean load over per-expert loads; 0 = balanced.

    [TD, summary] names maxvio as the deviation from the ideal distribution with 0 meaning
    perfect balance; its public benchmark sweeps maxvio 0.2..20 at EP=8, values a
    rank-level ratio cannot reach, so the loads are the per-expert token counts.
    """
    L = np.asarray(L, dtype=np.float64)
    mean = L.mean()
    return float((L.max() - mean) / mean)


@dataclasses.dataclass
class Entry:
    e: int      # replicated expert
    q: int      # rank that serves the replica
    a: int      # rows it serves
    j: int      # creation index among rank q's entries
    w: int      # weight row used on rank q: E+j (prefetch slot) or e (fallback to home row)


@dataclasses.dataclass
class Plan:
    R: int
    E: int
    B: int
    S: int
    K: int
    training: bool
    c: np.ndarray            # [R, E] counts
    L: np.ndarray            # [E] per-expert load
    P: np.ndarray            # [R] rows routed to each home group
    X: np.ndarray            # [R] P - S*K
    entries: List[Entry]     # in creation order
    keep: np.ndarray         # [E] rows of e served at its home rank
    n: np.ndarray            # [R, E+B] rows per weight row on each rank
    cu: np.ndarray           # [R, E+B+1] cu_seqlens
    instances: Dict[int, List[Tuple[int, int, int, int]]]  # e -> [(q, w, start, rows)]
    status: int

    @property
    def G(self) -> int:
        return self.E // self.R

    @property
    def C(self) -> int:
        return self.S * self.K


RULES = ("chain", "lowmig")


def make_plan(topk: np.ndarray, E: int, B: int, training: bool = False, rule: str = "chain") -> Plan:
    """Plan redundant experts so every rank serves exactly C = S*K rows.

    Steps (notation: G = E/R home experts per rank, h(e) = e // G its home rank):

    1. Counts.  L[e] rows want expert e; P[q] = rows wanting rank q's home group;
       X[q] = P[q] - C is rank q's excess (>0, a donor) or deficit (<0, a receiver).
       Sum of X is 0 because sum of P is R*C.
    2. Order.  Donors by excess descending, receivers by deficit descending; ties to
       the lower rank id.
    3. ship(d, t, amt) moves amt rows of donor d's home experts to rank t, one
       replica (expert, t) per piece: the expert of group d with the fewest remaining
       rows that still covers the whole amount (best fit), else the one with the most
       remaining rows, taking all of them; ties to the lower expert id.
    4. Chain.  Walk the donors in order.  A donor first repays the shortfall it
       inherited from the previous donor (see below), then covers whole receivers in
       order until its excess is used up.  Covering the last receiver whole can push
       the donor below C by some s rows; the next donor then ships those s rows to
       it.  So each receiver is fed by exactly one donor and each donor by at most
       the next one: at most one remote home group per rank [TC, Installation and
       integration].
    5. Slots.  On each rank the entries, in creation order, take prefetch slots
       E, E+1, ...; entries beyond the B slots read the home row e instead
       (fallback, counted) [TD, memory contract; TC, Installation and integration].
    6. Row counts and cu_seqlens per rank and weight row; every rank must total
       exactly C (the capacity check; the planner raises otherwise) [TC, text under
       Table 1].
    7. Instances.  Expert e is served first by its home rank (keep[e] rows), then by
       its replicas in creation order; the instance start offsets partition e's rows.

    ``rule="lowmig"`` replaces step 4 by a chain that moves fewer rows (fewer "migrated
    tokens" [TC, What we measured, Table 1]) under the same one-remote-group property:

    4'. Walk the donors in order; rem = the rows the donor must still ship.  A donor first
        repays a shortfall inherited from the previous donor, as in step 4.  The last donor
        then covers every receiver left.  Any other donor covers, again and again, the
        largest remaining receiver whose whole deficit fits in rem (ties to the lower
        rank).  When none fits and rem > 0, it either (a) covers the smallest remaining
        receiver whole (ties to the lower rank), falling s = deficit - rem rows short,
        which the next donor repays (step 4's carry, s rows moved twice), or (b) hands its
        rem rows to the next donor, which then ships rem more of its own (rem rows moved
        twice).  It takes (a) only when s < rem and it was handed no rows itself: a rank
        handed rows by the previous donor already serves that donor's group, and repaying
        would add the next donor's group.  Every rank still gets replicas from one ship
        call, so from at most one other home group.
    """
    topk = np.asarray(topk)
    validate_routing(topk, E)
    R, S, K = topk.shape
    if E % R != 0:
        raise ValueError("E must be a multiple of R")
    if B < 0:
        raise ValueError("B must be >= 0")
    G, C = E // R, S * K

    # 1. counts
    c, L = expert_counts(topk, E)
    P = np.array([int(L[q * G:(q + 1) * G].sum()) for q in range(R)], dtype=np.int64)
    X = P - C
    assert int(X.sum()) == 0

    # 2. order
    donors = sorted([q for q in range(R) if X[q] > 0], key=lambda q: (-X[q], q))
    receivers = sorted([q for q in range(R) if X[q] < 0], key=lambda q: (X[q], q))

    avail = [int(v) for v in L]
    raw: List[Tuple[int, int, int]] = []     # (e, q, a) in creation order

    # 3. ship
    def ship(d: int, t: int, amt: int) -> None:
        group = range(d * G, (d + 1) * G)
        while amt > 0:
            fits = [e for e in group if avail[e] >= amt]
            if fits:
                e = min(fits, key=lambda x: (avail[x], x))
            else:
                e = max(group, key=lambda x: (avail[x], -x))
            a = min(avail[e], amt)
            if a <= 0:
                raise CapacityError("donor group ran out of rows")
            raw.append((e, t, a))
            avail[e] -= a
            amt -= a

    if rule == "chain":
        # 4. chain
        j = 0
        carry = None          # (previous donor, rows it is short of C)
        for d in donors:
            rem = int(X[d])
            if carry is not None:
                t, s = carry
                ship(d, t, s)
                rem -= s
                carry = None
            while rem > 0 and j < len(receivers):
                t = receivers[j]
                need = int(-X[t])
                ship(d, t, need)
                rem -= need
                j += 1
            if rem < 0:
                carry = (d, -rem)
            elif rem > 0:
                raise CapacityError("excess left with no receiver")
        if carry is not None or j != len(receivers):
            raise CapacityError("chain did not close")
    elif rule == "lowmig":
        # 4'. packing chain with carries in either direction
        left = list(receivers)            # deficit desc, rank asc
        carry = None                      # (previous donor, rows it is short of C)
        handed = 0                        # rows the previous donor handed to this one
        for i, d in enumerate(donors):
            rem = int(X[d]) + handed
            may_repay = handed == 0
            handed = 0
            if carry is not None:
                t, s = carry
                ship(d, t, s)
                rem -= s
                carry = None
            if i == len(donors) - 1:
                for t in left:
                    ship(d, t, int(-X[t]))
                    rem += int(X[t])
                left = []
            while rem > 0 and left:
                fit = [t for t in left if -X[t] <= rem]
                if fit:
                    t = fit[0]
                    ship(d, t, int(-X[t]))
                    rem += int(X[t])
                    left.remove(t)
                    continue
                small = min(int(-X[t]) for t in left)
                t = next(t for t in left if -X[t] == small)
                if may_repay and small - rem < rem:
                    ship(d, t, small)         # (a) short by small - rem, repaid by the next donor
                    rem -= small
                    left.remove(t)
                else:
                    ship(d, donors[i + 1], rem)   # (b) the next donor ships these rows on
                    handed = rem
                    rem = 0
            if rem < 0:
                carry = (d, -rem)
            elif rem > 0:
                raise CapacityError("excess left with no receiver")
        if carry is not None or handed or left:
            raise CapacityError("chain did not close")
    else:
        raise ValueError(f"unknown plan rule {rule!r}")

    # 5. slots / fallback
    per_rank = [0] * R
    entries: List[Entry] = []
    for (e, q, a) in raw:
        jj = per_rank[q]
        per_rank[q] += 1
        w = E + jj if jj < B else e
        entries.append(Entry(e=e, q=q, a=a, j=jj, w=w))

    # 6. row counts, cu_seqlens, capacity check
    keep = np.array(avail, dtype=np.int64)
    n = np.zeros((R, E + B), dtype=np.int64)
    for e in range(E):
        n[e // G, e] += keep[e]
    for en in entries:
        n[en.q, en.w] += en.a
    cu = np.zeros((R, E + B + 1), dtype=np.int64)
    cu[:, 1:] = np.cumsum(n, axis=1)
    if np.any(cu[:, E + B] != C):
        raise CapacityError("a rank does not total S*K rows")

    # 7. instances
    instances: Dict[int, List[Tuple[int, int, int, int]]] = {}
    for e in range(E):
        lst = [(e // G, e, 0, int(keep[e]))]
        st = int(keep[e])
        for en in entries:
            if en.e == e:
                lst.append((en.q, en.w, st, en.a))
                st += en.a
        assert st == L[e]
        instances[e] = lst

    status = 0
    if training and any(en.w < E for en in entries):
        status |= ST_TRAIN_FALLBACK
    return Plan(R=R, E=E, B=B, S=S, K=K, training=training, c=c, L=L, P=P, X=X,
                entries=entries, keep=keep, n=n, cu=cu, instances=instances, status=status)


def destinations(topk: np.ndarray, plan: Plan) -> np.ndarray:
    """Final row of every (token, k) in the [R, S*K] receive buffer, computed on the send side.

    Zero-copy permute: the sender computes the receiver's final expert-grouped position and
    writes there, with no receive-then-sort step [TC, "What the technique is"; TD,
    architecture; AL, How it works].  Reading taken for the order inside a group: pairs of
    expert e are numbered g = 0 .. L[e]-1 in (rank, token) order; pair g goes to the
    instance whose [start, start + rows) holds g, at offset g - start inside that group.
    Groups inside a rank are ordered by weight row, as cu_seqlens lays them out.
    """
    R, S, K = topk.shape
    C = S * K
    dest = np.empty((R, S, K), dtype=np.int64)
    nxt = np.zeros(plan.E, dtype=np.int64)      # next g per expert
    for r in range(R):
        for s in range(S):
            for k in range(K):
                e = int(topk[r, s, k])
                g = int(nxt[e])
                nxt[e] += 1
                for (q, w, st, rows) in plan.instances[e]:
                    if st <= g < st + rows:
                        dest[r, s, k] = q * C + plan.cu[q, w] + (g - st)
                        break
                else:
                    raise CapacityError("pair outside every instance")
    return dest


def stats_vector(plan: Plan) -> np.ndarray:
    """The 16-word plan statistics (names in STAT_NAMES), as the library reports them.

    Replicas are the pages' "copy slots", migrated rows their "migrated tokens" [TC, What
    we measured, Table 1]; the migration bound is sum over ranks of max(0, X).
    """
    E, R = plan.E, plan.R
    slot = sum(1 for en in plan.entries if en.w >= E)
    fb = [en for en in plan.entries if en.w < E]
    per_rank = np.bincount([en.q for en in plan.entries], minlength=R) if plan.entries else np.zeros(R, int)
    v = np.zeros(16, dtype=np.int64)
    v[0] = plan.status
    v[1] = len(plan.entries)
    v[2] = slot
    v[3] = len(fb)
    v[4] = sum(en.a for en in fb)
    v[5] = sum(en.a for en in plan.entries)
    v[6] = int(np.maximum(plan.X, 0).sum())
    v[7] = int(plan.L.max())
    v[8] = int(plan.P.max())
    v[9] = int(plan.P.min())
    v[10] = int((plan.X > 0).sum())
    v[11] = int((plan.X < 0).sum())
    v[12] = int(per_rank.max()) if len(per_rank) else 0
    v[13] = int(plan.cu[:, -1].sum())
    return v
