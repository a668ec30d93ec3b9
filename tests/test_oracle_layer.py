"""Pins of the CPU oracle's permute, grouped SwiGLU FFN, unpermute and reduce_grad.

The grouped path (plan -> dispatch -> ffn -> combine, and its backward with
reduce_grad) is compared with the plan-free definition, and that definition
with torch's CPU autograd in float64 (an independent library routine).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W


def _layer(cfg, B=None):
    topk, gates, _ = W.routing_for(cfg)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, cfg.seed, cfg.dtype)
    w13, w2 = W.expert_weights_np(cfg.E, cfg.H, cfg.I, cfg.seed)
    plan = O.make_plan(topk, cfg.E, cfg.B if B is None else B, training=True)
    dest = O.destinations(topk, plan)
    return topk, gates, x, w13, w2, plan, dest


def _torch_moe(x, topk, gates, w13, w2):
    """Independent autograd reference in float64 on the CPU."""
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    W13 = torch.tensor(np.asarray(w13, np.float64), requires_grad=True)
    W2 = torch.tensor(np.asarray(w2, np.float64), requires_grad=True)
    I = w2.shape[1]
    R, S, K = topk.shape
    out = torch.zeros_like(xt)
    tk = torch.tensor(topk, dtype=torch.long)
    g = torch.tensor(np.asarray(gates, np.float64))
    for k in range(K):
        wk13 = W13[tk[:, :, k]]             # [R,S,H,2I]
        wk2 = W2[tk[:, :, k]]               # [R,S,I,H]
        h = torch.einsum("rsh,rshj->rsj", xt, wk13)
        a = torch.nn.functional.silu(h[..., :I]) * h[..., I:]
        y = torch.einsum("rsi,rsih->rsh", a, wk2)
        out = out + g[:, :, k:k + 1] * y
    return xt, W13, W2, out


def test_direct_forward_backward_vs_torch_autograd():
    cfg = W.CONFIGS["tiny"].with_(S=16, H=32, I=24)
    topk, gates, _ = W.routing_for(cfg)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, 1, "f32")
    w13, w2 = W.expert_weights_np(cfg.E, cfg.H, cfg.I, 1, std=0.2)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, 1, "f32")
    xt, W13, W2, out = _torch_moe(x, topk, gates, w13, w2)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    ref = O.moe_direct(x, topk, gates, w13, w2)
    np.testing.assert_allclose(ref, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    dx, dW13, dW2 = O.moe_direct_backward(x, topk, gates, w13, w2, dout)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW13, W13.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dW2, W2.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_silu_closed_form():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + np.exp(-1.0)))
    assert O.silu(np.array([-50.0]))[0] == pytest.approx(0.0, abs=1e-18)
    assert O.silu(np.array([50.0]))[0] == pytest.approx(50.0)


def test_dispatch_is_bitwise_and_writes_every_row_once():
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg)
    recv = O.dispatch(dest, x, fill=np.float32(np.nan))
    assert not np.isnan(recv).any()
    for r in range(cfg.R):
        for s in range(cfg.S):
            for k in range(cfg.K):
                assert recv[dest[r, s, k]].tobytes() == x[r, s].tobytes()
    xb = W.bf16_bits(x)
    rb = O.dispatch(dest, xb)
    assert rb.dtype == np.uint16 and np.array_equal(rb[dest[1, 5, 1]], xb[1, 5])


def test_combine_round_trip_identity_experts():
    """Identity experts (y = recv): out = sum_k g_k x = x because the gates sum to 1."""
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg)
    recv = O.dispatch(dest, x)
    out = O.combine(dest, recv, gates)
    np.testing.assert_allclose(out, x, rtol=2e-6, atol=2e-6)
    # unit gates: K copies of x
    np.testing.assert_allclose(O.combine(dest, recv, None), cfg.K * x.astype(np.float64), rtol=1e-12)


def test_combine_routing_tag():
    """Tag each received row with its weight row: the combine of token (r,s) must return
    sum_k g_k * (1 + T[r,s,k]) for an identity expert scaled by (1 + its expert id)."""
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg)
    ones = np.ones((cfg.R, cfg.S, 1))
    recv = O.dispatch(dest, ones)
    tag = np.full(cfg.R * cfg.C, -1.0)
    slot_e = {(en.q, en.w): en.e for en in plan.entries}
    for q in range(cfg.R):
        for w in range(cfg.E + cfg.B):
            lo, hi = q * cfg.C + plan.cu[q, w], q * cfg.C + plan.cu[q, w + 1]
            if hi > lo:
                tag[lo:hi] = 1 + (w if w < cfg.E else slot_e[(q, w)])
    out = O.combine(dest, recv * tag[:, None], gates)[:, :, 0]
    expect = (np.asarray(gates, np.float64) * (1 + topk)).sum(axis=2)
    np.testing.assert_allclose(out, expect, rtol=1e-6)


@pytest.mark.parametrize("B", [4, 2, 0])
def test_forward_replication_invariance(B):
    """Plan + dispatch + grouped FFN + combine equals the per-token definition (the pages:
    duplicates and fallback reads do not change the result)."""
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg, B=B)
    recv = O.dispatch(dest, x)
    s13, s2 = O.prefetch(plan, w13, w2)
    gu, act, y = O.ffn_forward(plan, recv, w13, w2, s13, s2)
    out = O.combine(dest, y, gates)
    ref = O.moe_direct(x, topk, gates, w13, w2)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("B", [4, 2, 0])
def test_backward_replication_invariance(B):
    """Grouped backward with reduce-buffer routing + reduce_grad equals the plan-free
    gradients; reduce_grad leaves the consumed slots zero."""
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg, B=B)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, cfg.seed, "f32")
    recv = O.dispatch(dest, x)
    s13, s2 = O.prefetch(plan, w13, w2)
    gu, act, y = O.ffn_forward(plan, recv, w13, w2, s13, s2)
    dy = O.dispatch(dest, dout, row_scale=gates)
    drecv, dW13, dW2, rb13, rb2 = O.ffn_backward(plan, recv, gu, act, dy, w13, w2, s13, s2)
    dx = O.combine(dest, drecv, None)
    O.reduce_grad(plan, dW13, dW2, rb13, rb2)
    rdx, rdW13, rdW2 = O.moe_direct_backward(x, topk, gates, w13, w2, dout)
    np.testing.assert_allclose(dx, rdx, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dW13, rdW13, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dW2, rdW2, rtol=1e-9, atol=1e-12)
    assert not rb13.any() and not rb2.any()
    if B == 0:
        assert all(en.w < cfg.E for en in plan.entries)


def test_reduce_grad_only_touches_slot_entries():
    cfg = W.CONFIGS["tiny"]
    topk, gates, x, w13, w2, plan, dest = _layer(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    dW13 = np.ones((E, H, 2 * I))
    dW2 = np.ones((E, I, H))
    rb13 = np.full((cfg.R, cfg.B, H, 2 * I), 2.0)
    rb2 = np.full((cfg.R, cfg.B, I, H), 2.0)
    O.reduce_grad(plan, dW13, dW2, rb13, rb2)
    used = {(en.q, en.j) for en in plan.entries if en.w >= E}
    n_rep = np.bincount([en.e for en in plan.entries if en.w >= E], minlength=E)
    for e in range(E):
        assert np.all(dW13[e] == 1 + 2 * n_rep[e])
    for q in range(cfg.R):
        for j in range(cfg.B):
            assert np.all(rb13[q, j] == (0.0 if (q, j) in used else 2.0))


def test_bf16_bits_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 3.0e38], dtype=np.float32)
    b = W.bf16_bits(v)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]
    assert W.bf16_to_f32(b)[0] == 1.0


def test_expert_and_token_helpers_vs_torch_autograd():
    """The per-expert weight gradient and the per-token output / input gradient (used where the
    whole layer is too large for the oracle) against torch's CPU autograd in float64."""
    cfg = W.CONFIGS["tiny"].with_(S=16, H=32, I=24)
    topk, gates, _ = W.routing_for(cfg)
    x = W.hidden_rows(cfg.R, cfg.S, cfg.H, 2, "f32")
    w13, w2 = W.expert_weights_np(cfg.E, cfg.H, cfg.I, 2, std=0.2)
    dout = W.grad_rows(cfg.R, cfg.S, cfg.H, 2, "f32")
    xt, W13, W2, out = _torch_moe(x, topk, gates, w13, w2)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    for e in (0, 3, cfg.E - 1):
        g13, g2, _ = O.expert_grad_direct(x, topk, gates, dout, e, w13[e], w2[e])
        np.testing.assert_allclose(g13, W13.grad.numpy()[e], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g2, W2.grad.numpy()[e], rtol=1e-10, atol=1e-12)
    toks = [(0, 0), (1, 5), (3, 15), (2, 7)]
    o, dx = O.token_grad_direct(x, topk, gates, dout, toks, lambda e: (w13[e], w2[e]))
    for i, (r, s) in enumerate(toks):
        np.testing.assert_allclose(o[i], out.detach().numpy()[r, s], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dx[i], xt.grad.numpy()[r, s], rtol=1e-10, atol=1e-12)
