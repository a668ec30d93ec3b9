"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from the seeded generator in ``workload``; expected values from the
CPU oracle in ``oracle``; the device results from the HIP library through its
Python binding.  Nothing here feeds a device result into the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import balanced_token_dispatch_moonep_amd as M
import oracle as O
import workload as W

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dims_of(cfg: W.Config, B=None, training=False, f32_rows=None, rule="chain") -> M.Dims:
    f32 = (cfg.dtype == "f32") if f32_rows is None else f32_rows
    return M.Dims.make(cfg.R, cfg.E, cfg.B if B is None else B, cfg.S, cfg.K, cfg.H, cfg.I,
                       training=training, f32_rows=f32, plan_rule=rule)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rows_tensor(x: np.ndarray) -> torch.Tensor:
    return bf16_from_bits(x) if x.dtype == np.uint16 else f32(x)


def run_plan(d: M.Dims, topk: np.ndarray, topk_dev=None):
    ws = torch.empty(M.moonep_plan_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    cu = torch.full((d.R, d.E + d.B + 1), -7, dtype=torch.int32, device=DEV)
    dest = torch.full((d.R, d.S, d.K), -7, dtype=torch.int32, device=DEV)
    stats = torch.full((M.NSTATS,), -7, dtype=torch.int32, device=DEV)
    tk = i32(topk) if topk_dev is None else topk_dev
    M.moonep_plan(d, tk, ws, cu, dest, stats)
    torch.cuda.synchronize()
    return ws, cu, dest, stats


def assert_plan_parity(d: M.Dims, topk: np.ndarray, training=False):
    """Bit-exact cu_seqlens, dest and stats against the oracle (the plan rule the dims' flags
    select); returns (oracle plan, dest, GPU tuple)."""
    rule = "lowmig" if d.flags & M.PLAN_LOWMIG else "chain"
    plan = O.make_plan(topk, d.E, d.B, training=training, rule=rule)
    dest = O.destinations(topk, plan)
    ws, cu, dd, st = run_plan(d, topk)
    np.testing.assert_array_equal(cu.cpu().numpy(), plan.cu)
    np.testing.assert_array_equal(dd.cpu().numpy(), dest)
    np.testing.assert_array_equal(st.cpu().numpy(), O.stats_vector(plan))
    return plan, dest, (ws, cu, dd, st)


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def max_row_rel(a: np.ndarray, b: np.ndarray) -> float:
    a2 = a.reshape(-1, a.shape[-1])
    b2 = b.reshape(-1, b.shape[-1])
    num = np.linalg.norm(a2 - b2, axis=1)
    den = np.maximum(np.linalg.norm(b2, axis=1), 1e-30)
    return float((num / den).max())
