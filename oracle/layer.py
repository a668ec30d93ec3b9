"""Oracle: permute, expert SwiGLU FFN over the plan's groups, unpermute, reduce_grad.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Page abbreviations as in
``oracle.plan``.  Floating point in float64; bf16 inputs arrive as uint16 bit
patterns and are widened exactly.

The numerical result the whole path must reproduce has a plain definition that
involves no plan at all (``moe_direct``): every token's output is the
gate-weighted sum of its K experts' SwiGLU FFNs.  Balancing does not change it:
duplicates and the home-row fallback are equally correct [TD, memory contract
and FAQ; TC, Installation and integration].  The grouped functions below
follow the path's own steps so each stage can be compared separately.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .plan import Plan


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:                       # bf16 bit patterns
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# permute / unpermute
# ----------------------------------------------------------------------------

def dispatch(dest: np.ndarray, x: np.ndarray, row_scale: Optional[np.ndarray] = None,
             fill=None) -> np.ndarray:
    """recv[dest[r,s,k]] = x[r,s]: each (token, k) row written straight into its final
    expert-grouped row of the [R*S*K, H] receive buffer [TC, "What the technique is";
    AL, How it works].

    Without ``row_scale`` the copy is bitwise (same dtype as ``x``).  With ``row_scale``
    ([R,S,K], the backward of a gate-weighted combine) the row is multiplied by its scale,
    in float64.
    """
    R, S, K = dest.shape
    H = x.shape[-1]
    if row_scale is None:
        recv = np.empty((R * S * K, H), dtype=x.dtype)
        if fill is not None:
            recv[...] = fill
        for r in range(R):
            for s in range(S):
                for k in range(K):
                    recv[dest[r, s, k]] = x[r, s]
        return recv
    xf = _f64(x)
    recv = np.zeros((R * S * K, H), dtype=np.float64)
    for r in range(R):
        for s in range(S):
            for k in range(K):
                recv[dest[r, s, k]] = float(row_scale[r, s, k]) * xf[r, s]
    return recv


def combine(dest: np.ndarray, y: np.ndarray, gates: Optional[np.ndarray] = None) -> np.ndarray:
    """out[r,s] = sum over k (in k order) of gates[r,s,k] * y[dest[r,s,k]]; unit gates if None.

    Gathers expert outputs back into token order [TC, flowchart "combine"].  Reading taken:
    the gather is gate-weighted, as the router's combine of a top-K MoE layer is.
    """
    R, S, K = dest.shape
    yf = _f64(y)
    out = np.zeros((R, S, yf.shape[-1]), dtype=np.float64)
    for k in range(K):
        g = np.ones((R, S)) if gates is None else np.asarray(gates[:, :, k], dtype=np.float64)
        out += g[:, :, None] * yf[dest[:, :, k]]
    return out


# ----------------------------------------------------------------------------
# groups and weight rows
# ----------------------------------------------------------------------------

def groups(plan: Plan) -> List[Tuple[int, int, int, int, str, int]]:
    """Non-empty GEMM groups: (q, w, first absolute row, rows, kind, index).

    Group (q, w) holds rows cu[q][w] .. cu[q][w+1]-1 of rank q's partition and uses weight
    row w of the [E+B, H, H'] tensor [TD, memory contract; TC, Installation and
    integration].  kind: 'home' (w < E, rank q owns e = w), 'fallback' (w < E, another
    rank's expert read from its home row), 'slot' (w >= E, prefetch slot w - E).
    """
    E, G, C = plan.E, plan.G, plan.C
    out = []
    for q in range(plan.R):
        for w in range(E + plan.B):
            rows = int(plan.n[q, w])
            if rows == 0:
                continue
            row0 = q * C + int(plan.cu[q, w])
            if w >= E:
                out.append((q, w, row0, rows, "slot", w - E))
            elif w // G == q:
                out.append((q, w, row0, rows, "home", w))
            else:
                out.append((q, w, row0, rows, "fallback", w))
    return out


def prefetch(plan: Plan, w13: np.ndarray, w2: np.ndarray):
    """Copy each slotted replica's home weights into its rank's prefetch slot.

    Slot (q, j) receives W[e] for the entry (e, q) with creation index j < B [TC, flowchart
    "Weight prefetch"; TD, memory contract].  Unused slots are zero here.
    """
    R, B = plan.R, plan.B
    s13 = np.zeros((R, B) + w13.shape[1:], dtype=w13.dtype)
    s2 = np.zeros((R, B) + w2.shape[1:], dtype=w2.dtype)
    for en in plan.entries:
        if en.w >= plan.E:
            s13[en.q, en.j] = w13[en.e]
            s2[en.q, en.j] = w2[en.e]
    return s13, s2


def _weights(plan: Plan, q: int, w: int, w13, w2, s13, s2):
    if w < plan.E:
        return _f64(w13[w]), _f64(w2[w])
    return _f64(s13[q, w - plan.E]), _f64(s2[q, w - plan.E])


# ----------------------------------------------------------------------------
# expert FFN over groups
# ----------------------------------------------------------------------------

def swiglu_ffn(X: np.ndarray, W13: np.ndarray, W2: np.ndarray):
    """One expert's SwiGLU FFN on rows X, float64: Gt = X W1, U = X W3 (W13 = [W1 | W3]),
    A = silu(Gt) * U, Y = A W2 [TC, flowchart "Group GEMM"; TC, What we measured, Table 2:
    three projections].  bf16 inputs arrive as uint16 bit patterns and are widened exactly.
    Returns (gu = [Gt | U], A, Y)."""
    X, W13, W2 = _f64(X), _f64(W13), _f64(W2)
    I = W2.shape[0]
    g = X @ W13
    a = silu(g[:, :I]) * g[:, I:]
    return g, a, a @ W2


def swiglu_ffn_backward(X: np.ndarray, gu: np.ndarray, act: np.ndarray, dY: np.ndarray,
                        W13: np.ndarray, W2: np.ndarray):
    """Backward of ``swiglu_ffn`` for upstream dY, float64.

    dA = dY W2^T; dGt = dA * U * sig(Gt) * (1 + Gt (1 - sig(Gt))); dU = dA * silu(Gt);
    dX = [dGt dU] W13^T; dW13 = X^T [dGt dU]; dW2 = A^T dY.
    Returns (dgu = [dGt | dU], dX, dW13, dW2)."""
    I = W2.shape[0]
    gt, u = gu[:, :I], gu[:, I:]
    da = dY @ W2.T
    sg = _sigmoid(gt)
    dgu = np.concatenate([da * u * sg * (1.0 + gt * (1.0 - sg)), da * silu(gt)], axis=1)
    return dgu, dgu @ W13.T, X.T @ dgu, act.T @ dY


def ffn_forward(plan: Plan, recv, w13, w2, s13, s2):
    """Grouped SwiGLU FFN on the receive buffer, group by group.

    For group rows X_g with weight row w: Gt = X_g W1, U = X_g W3, A = silu(Gt) * U,
    Y_g = A W2, silu(x) = x / (1 + exp(-x)) [TC, flowchart "Group GEMM"; TD, memory
    contract].  Returns (gu [R*C, 2I] = [Gt | U], act [R*C, I], y [R*C, H]) in float64.
    """
    X = _f64(recv)
    I = w2.shape[1]
    M, H = X.shape
    gu = np.zeros((M, 2 * I))
    act = np.zeros((M, I))
    y = np.zeros((M, H))
    for (q, w, row0, rows, kind, idx) in groups(plan):
        W13, W2 = _weights(plan, q, w, w13, w2, s13, s2)
        sl = slice(row0, row0 + rows)
        gu[sl], act[sl], y[sl] = swiglu_ffn(X[sl], W13, W2)
    return gu, act, y


def ffn_backward(plan: Plan, recv, gu, act, dy, w13, w2, s13, s2):
    """Backward of ``ffn_forward`` with the replica-gradient routing.

    dA = dY W2^T; dGt = dA * U * sig(Gt) * (1 + Gt (1 - sig(Gt))); dU = dA * silu(Gt);
    dX_g = [dGt dU] W13^T; dW2_g = A^T dY; dW13_g = X_g^T [dGt dU].

    Weight gradients of prefetched replicas go to a separate fp32 reduce buffer
    RB[q, j] instead of the parameter gradients [TD, memory contract; AT, Technical
    Details].  Home groups add into dW_home[e].  Fallback groups (a replica that had no
    slot, B < E/R) add into dW_home[e] after the home group, in entry order; the pages
    require B = E/R for training, so this last case is an extension with the same
    result as an all-home computation.

    Returns (drecv [R*C, H], dW13_home [E,H,2I], dW2_home [E,I,H], RB13 [R,B,H,2I],
    RB2 [R,B,I,H]) in float64, starting from zero.
    """
    X = _f64(recv)
    GU = _f64(gu)
    A = _f64(act)
    DY = _f64(dy)
    E, R, B = plan.E, plan.R, plan.B
    H, I2 = w13.shape[1], w13.shape[2]
    I = I2 // 2
    drecv = np.zeros_like(X)
    dW13 = np.zeros((E, H, I2))
    dW2 = np.zeros((E, I, H))
    rb13 = np.zeros((R, B, H, I2))
    rb2 = np.zeros((R, B, I, H))
    grp = groups(plan)
    order = [g for g in grp if g[4] == "home"] + [g for g in grp if g[4] == "slot"]
    fb = {(en.q, en.w): i for i, en in enumerate(plan.entries) if en.w < E}
    order += sorted([g for g in grp if g[4] == "fallback"], key=lambda g: fb[(g[0], g[1])])
    for (q, w, row0, rows, kind, idx) in order:
        W13, W2 = _weights(plan, q, w, w13, w2, s13, s2)
        sl = slice(row0, row0 + rows)
        _, drecv[sl], g13, g2 = swiglu_ffn_backward(X[sl], GU[sl], A[sl], DY[sl], W13, W2)
        if kind == "slot":
            rb13[q, idx] += g13
            rb2[q, idx] += g2
        else:
            dW13[w] += g13
            dW2[w] += g2
    return drecv, dW13, dW2, rb13, rb2


def reduce_grad(plan: Plan, dW13, dW2, rb13, rb2) -> None:
    """Fold replica gradients into the home experts' gradients and clear the used slots.

    For every expert, its prefetched replicas' reduce-buffer slots are added, in creation
    order, to the expert's parameter gradient, then zeroed for the next micro-batch [TD,
    memory contract; AT, Technical Details].  In place.
    """
    for en in plan.entries:          # creation order
        if en.w >= plan.E:
            dW13[en.e] += rb13[en.q, en.j]
            dW2[en.e] += rb2[en.q, en.j]
            rb13[en.q, en.j] = 0.0
            rb2[en.q, en.j] = 0.0


# ----------------------------------------------------------------------------
# plain definition (no plan)
# ----------------------------------------------------------------------------

def moe_direct(x, topk, gates, w13, w2) -> np.ndarray:
    """out[r,s] = sum_k gates[r,s,k] * FFN_{topk[r,s,k]}(x[r,s]), float64, no plan involved."""
    xf = _f64(x)
    R, S, H = xf.shape
    E = w13.shape[0]
    out = np.zeros((R, S, H))
    for e in range(E):
        r_i, s_i, k_i = np.nonzero(topk == e)
        if r_i.size == 0:
            continue
        _, _, ye = swiglu_ffn(xf[r_i, s_i], _f64(w13[e]), _f64(w2[e]))
        np.add.at(out, (r_i, s_i), np.asarray(gates, np.float64)[r_i, s_i, k_i][:, None] * ye)
    return out


def expert_grad_direct(x, topk, gates, dout, e: int, W13, W2):
    """Plan-free gradient of expert e's weights: every (token, k) routed to e contributes,
    whichever rank serves it, with upstream gradient gates[r,s,k] * dOut[r,s] (float64).

    ``W13`` [H, 2I] and ``W2`` [I, H] are expert e's weights.  Returns (dW13_e, dW2_e, rows of
    dx contributed by e as (r_i, s_i, dx_rows))."""
    xf = _f64(x)
    r_i, s_i, k_i = np.nonzero(topk == e)
    W13f, W2f = _f64(W13), _f64(W2)
    if r_i.size == 0:
        return (np.zeros(W13f.shape), np.zeros(W2f.shape), (r_i, s_i, np.zeros((0, xf.shape[-1]))))
    xe = xf[r_i, s_i]
    gu, a, _ = swiglu_ffn(xe, W13f, W2f)
    dy = np.asarray(gates, np.float64)[r_i, s_i, k_i][:, None] * _f64(dout[r_i, s_i])
    _, dxe, dW13, dW2 = swiglu_ffn_backward(xe, gu, a, dy, W13f, W2f)
    return dW13, dW2, (r_i, s_i, dxe)


def moe_direct_backward(x, topk, gates, w13, w2, dout, experts=None):
    """Gradients of ``moe_direct`` w.r.t. x, W13 and W2 for upstream dOut (float64).

    ``experts`` restricts the computation to those experts (dx then only holds their share).
    """
    xf = _f64(x)
    E = w13.shape[0]
    dx = np.zeros_like(xf)
    dW13 = np.zeros((E,) + tuple(w13.shape[1:]))
    dW2 = np.zeros((E,) + tuple(w2.shape[1:]))
    for e in (range(E) if experts is None else experts):
        dW13[e], dW2[e], (r_i, s_i, dxe) = expert_grad_direct(xf, topk, gates, dout, e, w13[e], w2[e])
        np.add.at(dx, (r_i, s_i), dxe)
    return dx, dW13, dW2


def token_grad_direct(x, topk, gates, dout, tokens, weights_of):
    """Plan-free output and input gradient of a few tokens: for each (r, s) in ``tokens``,
    out[r,s] = sum_k g_k FFN_{e_k}(x[r,s]) and dx[r,s] = sum_k of the gradient of g_k FFN_{e_k}
    at x[r,s] for upstream dOut[r,s], both in k order (float64).  ``weights_of(e)`` returns
    expert e's (W13 [H, 2I], W2 [I, H]), so only the experts of these tokens are read.
    Returns (out [n, H], dx [n, H])."""
    xf = _f64(np.asarray([x[r, s] for (r, s) in tokens]))
    do = _f64(np.asarray([dout[r, s] for (r, s) in tokens]))
    out = np.zeros(xf.shape)
    dx = np.zeros(xf.shape)
    for i, (r, s) in enumerate(tokens):
        for k in range(topk.shape[2]):
            W13, W2 = (_f64(w) for w in weights_of(int(topk[r, s, k])))
            g = float(gates[r, s, k])
            xi = xf[i:i + 1]
            gu, a, y = swiglu_ffn(xi, W13, W2)
            out[i] += g * y[0]
            _, dxi, _, _ = swiglu_ffn_backward(xi, gu, a, g * do[i:i + 1], W13, W2)
            dx[i] += dxi[0]
    return out, dx
