"""Oracle: per-rank buffer sizes of the memory contract, in bytes.  TEST INFRASTRUCTURE ONLY.

[TD, memory contract] fixes the shapes: a [E+B, H, H'] weight tensor per expert
projection, whose rows [E, E+B) are B prefetch slots; an fp32 gradient buffer
of the same layout whose slot rows form the [R, B, H, H'] reduce view; a
static S*K-row dispatch buffer.  [TC, What we measured, Table 2] prices them
with three projections, S=4096, H=7168, H'=2048, bf16 weights and activations.
"""
from __future__ import annotations


def buffer_bytes(B: int, S: int, K: int, H: int, I: int, E_home: int = 0,
                 projections: int = 3, act_bytes: int = 2, w_bytes: int = 2,
                 grad_bytes: int = 4, training: bool = False) -> dict:
    """Per-rank bytes: prefetch slots, fp32 reduce buffer (training), dispatch buffer, home weights."""
    per_expert = projections * H * I
    out = {
        "prefetch": B * per_expert * w_bytes,
        "reduce": B * per_expert * grad_bytes if training else 0,
        "dispatch": S * K * H * act_bytes,
        "home_weights": E_home * per_expert * w_bytes,
    }
    out["total"] = out["prefetch"] + out["reduce"] + out["dispatch"]
    return out
