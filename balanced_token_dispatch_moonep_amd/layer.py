"""Static-shape buffers and call order for one balanced expert-parallel MoE layer.

The MoonEP pages describe one pass as: router output -> planning -> (weight prefetch
and dispatch) -> grouped GEMM -> combine, then reduce_grad of replica gradients in
training [thakicloud.com "The Busiest Rank Sets Your Step Time", "What the technique
is" flowchart].  Every buffer has a fixed shape (the receive buffer is always S*K rows
per rank), so it is allocated once and reused each step with no host synchronisation
[twodots.gr "MoonEP balances AI experts in MoE models", architecture].

This module only allocates device memory through torch and calls the library's entry
points in that order; all arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import (Dims, moonep_combine, moonep_dispatch, moonep_grouped_ffn,
               moonep_grouped_ffn_backward, moonep_plan, moonep_plan_workspace_bytes,
               moonep_prefetch, moonep_reduce_grad, NSTATS)


def _slot_shapes(R, B, H, I):
    return (R, B, H, 2 * I), (R, B, I, H)


def _nbytes(shape, itemsize):
    n = itemsize
    for v in shape:
        n *= v
    return n


class MoonEPPool:
    """Process-global prefetch slots shared by every layer [AT, TL;DR; TD, memory contract].

    Layers run one after another, so one set of B weight slots per rank (and, in training,
    one fp32 reduce buffer [R, B, ...]) serves all of them: the extra memory does not grow
    with depth.  A layer whose slots were overwritten by later layers prefetches its replicas
    again before its backward (its plan stays in its own workspace).
    """

    def __init__(self, R, B, H, I, training=False, device="cuda"):
        dev = torch.device(device)
        s13, s2 = _slot_shapes(R, B, H, I)
        self.R, self.B, self.H, self.I, self.training = R, B, H, I, training
        self.w13_slot = torch.zeros(s13, dtype=torch.bfloat16, device=dev) if B else None
        self.w2_slot = torch.zeros(s2, dtype=torch.bfloat16, device=dev) if B else None
        self.dw13_red = torch.zeros(s13, dtype=torch.float32, device=dev) if B and training else None
        self.dw2_red = torch.zeros(s2, dtype=torch.float32, device=dev) if B and training else None
        self.owner = None     # the layer whose replicas the slots hold

    @staticmethod
    def nbytes(R, B, H, I, training=False) -> dict:
        s13, s2 = _slot_shapes(R, B, H, I)
        slots = _nbytes(s13, 2) + _nbytes(s2, 2) if B else 0
        red = _nbytes(s13, 4) + _nbytes(s2, 4) if B and training else 0
        return {"prefetch": slots, "reduce": red, "total": slots + red}


def stack_slot_bytes(R, B, H, I, layers, pooled, training=False) -> int:
    """Bytes of prefetch slots (and reduce buffers) for `layers` layers, pooled or one set each."""
    per = MoonEPPool.nbytes(R, B, H, I, training)["total"]
    return per if pooled else layers * per


class MoonEPLayer:
    """One emulated EP layer: R ranks as R static partitions of one GPU's memory.

    ``w13`` [E, H, 2I] and ``w2`` [E, I, H] are the home expert weights (bf16, on the
    device).  With ``I == 0`` the layer has no expert FFN (identity experts): only
    planning, dispatch and combine run.
    """

    def __init__(self, dims: Dims, w13=None, w2=None, training: bool = False, device="cuda", pool=None):
        self.d = dims
        self.training = training
        self.pool = pool
        dev = torch.device(device)
        self.device = dev
        R, E, B, S, K, H, I = dims.R, dims.E, dims.B, dims.S, dims.K, dims.H, dims.I
        M = R * S * K
        rt = torch.float32 if dims.flags & 2 else torch.bfloat16
        i32 = torch.int32
        self.ws = torch.empty(moonep_plan_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        self.cu = torch.empty((R, E + B + 1), dtype=i32, device=dev)
        self.dest = torch.empty((R, S, K), dtype=i32, device=dev)
        self.stats = torch.empty((NSTATS,), dtype=i32, device=dev)
        self.recv = torch.empty((M, H), dtype=rt, device=dev)
        self.out = torch.empty((R, S, H), dtype=rt, device=dev)
        self.w13, self.w2 = w13, w2
        if I > 0:
            bf = torch.bfloat16
            if pool is not None:
                if (pool.R, pool.B, pool.H, pool.I) != (R, B, H, I) or (training and not pool.training):
                    raise ValueError("the pool's shapes do not match the layer")
                self.w13_slot, self.w2_slot = pool.w13_slot, pool.w2_slot
            else:
                self.w13_slot = torch.zeros((R, B, H, 2 * I), dtype=bf, device=dev) if B else None
                self.w2_slot = torch.zeros((R, B, I, H), dtype=bf, device=dev) if B else None
            self.gu = torch.empty((M, 2 * I), dtype=bf, device=dev)
            self.act = torch.empty((M, I), dtype=bf, device=dev)
            self.y = torch.empty((M, H), dtype=bf, device=dev)
            if training:
                f32 = torch.float32
                self.dy = torch.empty((M, H), dtype=bf, device=dev)
                self.drecv = torch.empty((M, H), dtype=bf, device=dev)
                self.dx = torch.empty((R, S, H), dtype=bf, device=dev)
                self.dw13 = torch.zeros((E, H, 2 * I), dtype=f32, device=dev)
                self.dw2 = torch.zeros((E, I, H), dtype=f32, device=dev)
                if pool is not None:
                    self.dw13_red, self.dw2_red = pool.dw13_red, pool.dw2_red
                else:
                    self.dw13_red = torch.zeros((R, B, H, 2 * I), dtype=f32, device=dev) if B else None
                    self.dw2_red = torch.zeros((R, B, I, H), dtype=f32, device=dev) if B else None
        else:
            self.y = self.recv          # identity experts

    # -- steps ---------------------------------------------------------------
    def plan(self, topk):
        moonep_plan(self.d, topk, self.ws, self.cu, self.dest, self.stats)

    def prefetch(self):
        if self.d.I > 0 and self.d.B > 0:
            moonep_prefetch(self.d, self.ws, self.w13, self.w2, self.w13_slot, self.w2_slot)
            if self.pool is not None:
                self.pool.owner = self

    def dispatch(self, x):
        moonep_dispatch(self.d, self.dest, x, None, self.recv)

    def expert_ffn(self):
        if self.d.I > 0:
            moonep_grouped_ffn(self.d, self.ws, self.cu, self.recv, self.w13, self.w2,
                               self.w13_slot, self.w2_slot, self.gu, self.act, self.y)

    def combine(self, gates):
        moonep_combine(self.d, self.dest, self.y, gates, self.out)

    def forward(self, x, topk, gates):
        """Returns the [R, S, H] output (a view of a static buffer, replaced by the next call)."""
        self.plan(topk)
        self.prefetch()
        self.dispatch(x)
        self.expert_ffn()
        self.combine(gates)
        return self.out

    def backward(self, dout, gates):
        """Gradient of forward(): returns dx [R, S, H]; writes dw13 / dw2 (fp32; added to them
        with MOONEP_GRAD_ACCUM), slot replicas' gradients reduced into their home experts.

        The saved gate|up activations are overwritten by their gradients."""
        assert self.training and self.d.I > 0
        if self.pool is not None and self.pool.owner is not self:
            self.prefetch()       # a later layer reused the shared slots
        moonep_dispatch(self.d, self.dest, dout, gates, self.dy)
        moonep_grouped_ffn_backward(self.d, self.ws, self.cu, self.recv, self.gu, self.act, self.dy,
                                    self.w13, self.w2, self.w13_slot, self.w2_slot, self.drecv,
                                    self.dw13, self.dw2, self.dw13_red, self.dw2_red)
        moonep_combine(self.d, self.dest, self.drecv, None, self.dx)
        moonep_reduce_grad(self.d, self.ws, self.dw13, self.dw2, self.dw13_red, self.dw2_red)
        return self.dx
