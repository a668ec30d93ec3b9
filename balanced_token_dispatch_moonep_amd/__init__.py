"""Python binding of libmoonep.so, the MoonEP balanced expert-parallel hot path on MI355X.

Thin ctypes marshalling only: every function here checks tensor shapes, dtypes,
devices and contiguity, then passes raw device pointers and the current HIP
stream to the C entry point of the same name (declared in include/moonep.h).
Tensors must live on the current device, and an explicit stream must belong to it.
All computation happens in the library's HIP kernels; there is no Python or
CPU fallback, and importing this package fails loudly if the library was not
built (``python -m balanced_token_dispatch_moonep_amd.build``).

PyTorch is used only to own device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MoonEPError", "Dims", "LIB_PATH", "lib", "NSTATS", "STAT_NAMES", "TRAINING", "F32_ROWS", "GRAD_ACCUM",
    "PLAN_LOWMIG",
    "PHASE_GATE_UP", "PHASE_DOWN", "PHASE_DACT", "PHASE_DX", "PHASE_DW2", "PHASE_DW13",
    "ST_BAD_ID", "ST_DUP_ID", "ST_CAPACITY", "ST_OVERFLOW", "ST_TRAIN_FALLBACK",
    "moonep_plan_workspace_bytes", "moonep_plan", "moonep_plan_noalloc", "NOALLOC_WS_BYTES",
    "moonep_prefetch", "moonep_dispatch",
    "moonep_combine", "moonep_dispatch_staged", "moonep_combine_staged", "moonep_grouped_ffn",
    "moonep_grouped_ffn_backward", "moonep_reduce_grad", "moonep_strerror", "moonep_version", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoonep.so")

TRAINING = 1
F32_ROWS = 2
GRAD_ACCUM = 4
PLAN_LOWMIG = 512      # the planner's low-migration rule
# phase selection of the expert FFN calls (one GEMM kernel each; none set = all of the call's)
PHASE_GATE_UP, PHASE_DOWN = 8, 16
PHASE_DACT, PHASE_DX, PHASE_DW2, PHASE_DW13 = 32, 64, 128, 256
NSTATS = 16
ST_BAD_ID, ST_DUP_ID, ST_CAPACITY, ST_OVERFLOW, ST_TRAIN_FALLBACK = 1, 2, 4, 8, 16
STAT_NAMES = (
    "status", "replicas", "slot_replicas", "fallback_replicas", "fallback_rows",
    "migrated_rows", "migration_bound", "max_expert_load", "max_rank_load",
    "min_rank_load", "donors", "receivers", "max_replicas_per_rank", "total_rows",
    "reserved14", "reserved15",
)
NOALLOC_WS_BYTES = 8 << 20     # static plan workspace of moonep_plan_noalloc, per GPU
EXPORTED = (
    "moonep_plan_workspace_bytes", "moonep_plan", "moonep_plan_noalloc", "moonep_prefetch", "moonep_dispatch",
    "moonep_combine", "moonep_dispatch_staged", "moonep_combine_staged", "moonep_grouped_ffn",
    "moonep_grouped_ffn_backward", "moonep_reduce_grad", "moonep_strerror", "moonep_version",
)


class MoonEPError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {moonep_strerror(code)} ({code})")
        self.code = code


class Dims(ctypes.Structure):
    """moonep_dims_t."""
    _fields_ = [("R", ctypes.c_int32), ("E", ctypes.c_int32), ("B", ctypes.c_int32),
                ("S", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    @classmethod
    def make(cls, R, E, B, S, K, H, I=0, training=False, f32_rows=False, grad_accum=False, phases=0,
             plan_rule="chain") -> "Dims":
        if plan_rule not in ("chain", "lowmig"):
            raise ValueError(f"unknown plan rule {plan_rule!r}")
        flags = (TRAINING if training else 0) | (F32_ROWS if f32_rows else 0) | (GRAD_ACCUM if grad_accum else 0)
        flags |= int(phases) | (PLAN_LOWMIG if plan_rule == "lowmig" else 0)
        return cls(R, E, B, S, K, H, I, flags)

    def with_flags(self, flags: int) -> "Dims":
        return Dims(self.R, self.E, self.B, self.S, self.K, self.H, self.I, int(flags))

    @property
    def C(self) -> int:
        return self.S * self.K


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m balanced_token_dispatch_moonep_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.moonep_plan_workspace_bytes.argtypes = [P]
    L.moonep_plan_workspace_bytes.restype = SZ
    L.moonep_plan.argtypes = [P, VP, VP, VP, VP, VP, VP]
    L.moonep_plan_noalloc.argtypes = [P, VP, VP, VP, VP, VP]
    L.moonep_prefetch.argtypes = [P, VP, VP, VP, VP, VP, VP]
    L.moonep_dispatch.argtypes = [P, VP, VP, VP, VP, VP]
    L.moonep_combine.argtypes = [P, VP, VP, VP, VP, VP]
    L.moonep_dispatch_staged.argtypes = [P, VP, VP, VP, VP, VP, VP]
    L.moonep_combine_staged.argtypes = [P, VP, VP, VP, VP, VP, VP]
    L.moonep_grouped_ffn.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP]
    L.moonep_grouped_ffn_backward.argtypes = [P] + [VP] * 16
    L.moonep_reduce_grad.argtypes = [P, VP, VP, VP, VP, VP, VP]
    for n in ("moonep_plan", "moonep_plan_noalloc", "moonep_prefetch", "moonep_dispatch", "moonep_combine",
              "moonep_dispatch_staged", "moonep_combine_staged", "moonep_grouped_ffn",
              "moonep_grouped_ffn_backward", "moonep_reduce_grad"):
        getattr(L, n).restype = I32
    L.moonep_strerror.argtypes = [I32]
    L.moonep_strerror.restype = ctypes.c_char_p
    L.moonep_version.argtypes = []
    L.moonep_version.restype = ctypes.c_char_p
    return L


_LIB = None


def _lib():
    """The loaded library (loaded on first use; raises ImportError if it was never built)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def moonep_strerror(code: int) -> str:
    return _lib().moonep_strerror(int(code)).decode()


def moonep_version() -> str:
    return _lib().moonep_version().decode()


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream) if isinstance(stream, int) else int(stream.cuda_stream)
    torch = _torch()
    return int(torch.cuda.current_stream().cuda_stream)


def _ptr(t, name, dtype=None, shape=None, numel=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the library runs on the current device "
                         f"cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _ws(d: Dims, plan_ws):
    """The plan workspace: uint8, exactly moonep_plan_workspace_bytes(d) bytes."""
    return _ptr(plan_ws, "plan_ws", _torch().uint8, numel=moonep_plan_workspace_bytes(d))


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise MoonEPError(rc, where)


def _rows_dtype(d: Dims):
    torch = _torch()
    return torch.float32 if d.flags & F32_ROWS else torch.bfloat16


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def moonep_plan_workspace_bytes(d: Dims) -> int:
    n = _lib().moonep_plan_workspace_bytes(ctypes.byref(d))
    if n == 0:
        raise MoonEPError(-1, "moonep_plan_workspace_bytes")
    return int(n)


def moonep_plan(d: Dims, topk, plan_ws, cu_seqlens, dest, stats, stream=None) -> None:
    torch = _torch()
    args = (
        _ptr(topk, "topk", torch.int32, (d.R, d.S, d.K)),
        _ws(d, plan_ws),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (d.R, d.E + d.B + 1)),
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(stats, "stats", torch.int32, (NSTATS,)),
    )
    _check(_lib().moonep_plan(ctypes.byref(d), *args, _stream(stream)), "moonep_plan")


def moonep_plan_noalloc(d: Dims, topk, cu_seqlens, dest, stats, stream=None) -> None:
    """moonep_plan with the library's static plan workspace (no device allocation); for the
    plan + dispatch + combine path.  Calls overlapping on one GPU race."""
    torch = _torch()
    args = (
        _ptr(topk, "topk", torch.int32, (d.R, d.S, d.K)),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (d.R, d.E + d.B + 1)),
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(stats, "stats", torch.int32, (NSTATS,)),
    )
    _check(_lib().moonep_plan_noalloc(ctypes.byref(d), *args, _stream(stream)), "moonep_plan_noalloc")


def moonep_prefetch(d: Dims, plan_ws, w13_home, w2_home, w13_slot, w2_slot, stream=None) -> None:
    torch = _torch()
    bf = torch.bfloat16
    args = (
        _ws(d, plan_ws),
        _ptr(w13_home, "w13_home", bf, (d.E, d.H, 2 * d.I)),
        _ptr(w2_home, "w2_home", bf, (d.E, d.I, d.H)),
        _ptr(w13_slot, "w13_slot", bf, (d.R, d.B, d.H, 2 * d.I), optional=d.B == 0),
        _ptr(w2_slot, "w2_slot", bf, (d.R, d.B, d.I, d.H), optional=d.B == 0),
    )
    _check(_lib().moonep_prefetch(ctypes.byref(d), *args, _stream(stream)), "moonep_prefetch")


def moonep_dispatch(d: Dims, dest, src, row_scale, recv, stream=None) -> None:
    torch = _torch()
    rt = _rows_dtype(d)
    args = (
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(src, "src", rt, (d.R, d.S, d.H)),
        _ptr(row_scale, "row_scale", torch.float32, (d.R, d.S, d.K), optional=True),
        _ptr(recv, "recv", rt, (d.R * d.S * d.K, d.H)),
    )
    _check(_lib().moonep_dispatch(ctypes.byref(d), *args, _stream(stream)), "moonep_dispatch")


def moonep_combine(d: Dims, dest, y, gates, out, stream=None) -> None:
    torch = _torch()
    rt = _rows_dtype(d)
    args = (
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(y, "y", rt, (d.R * d.S * d.K, d.H)),
        _ptr(gates, "gates", torch.float32, (d.R, d.S, d.K), optional=True),
        _ptr(out, "out", rt, (d.R, d.S, d.H)),
    )
    _check(_lib().moonep_combine(ctypes.byref(d), *args, _stream(stream)), "moonep_combine")


def moonep_dispatch_staged(d: Dims, dest, src, row_scale, stage, recv, stream=None) -> None:
    """Non-zero-copy baseline of moonep_dispatch (arrival-order copy, then a sort-copy)."""
    torch = _torch()
    rt = _rows_dtype(d)
    M = d.R * d.S * d.K
    args = (
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(src, "src", rt, (d.R, d.S, d.H)),
        _ptr(row_scale, "row_scale", torch.float32, (d.R, d.S, d.K), optional=True),
        _ptr(stage, "stage", rt, (M, d.H)),
        _ptr(recv, "recv", rt, (M, d.H)),
    )
    _check(_lib().moonep_dispatch_staged(ctypes.byref(d), *args, _stream(stream)), "moonep_dispatch_staged")


def moonep_combine_staged(d: Dims, dest, y, gates, stage, out, stream=None) -> None:
    """Non-zero-copy baseline of moonep_combine (gather to arrival order, then reduce)."""
    torch = _torch()
    rt = _rows_dtype(d)
    M = d.R * d.S * d.K
    args = (
        _ptr(dest, "dest", torch.int32, (d.R, d.S, d.K)),
        _ptr(y, "y", rt, (M, d.H)),
        _ptr(gates, "gates", torch.float32, (d.R, d.S, d.K), optional=True),
        _ptr(stage, "stage", rt, (M, d.H)),
        _ptr(out, "out", rt, (d.R, d.S, d.H)),
    )
    _check(_lib().moonep_combine_staged(ctypes.byref(d), *args, _stream(stream)), "moonep_combine_staged")


def moonep_grouped_ffn(d: Dims, plan_ws, cu_seqlens, recv, w13_home, w2_home, w13_slot, w2_slot,
                       gu_save, act, y, stream=None) -> None:
    torch = _torch()
    bf = torch.bfloat16
    M = d.R * d.S * d.K
    args = (
        _ws(d, plan_ws),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (d.R, d.E + d.B + 1)),
        _ptr(recv, "recv", bf, (M, d.H)),
        _ptr(w13_home, "w13_home", bf, (d.E, d.H, 2 * d.I)),
        _ptr(w2_home, "w2_home", bf, (d.E, d.I, d.H)),
        _ptr(w13_slot, "w13_slot", bf, (d.R, d.B, d.H, 2 * d.I), optional=d.B == 0),
        _ptr(w2_slot, "w2_slot", bf, (d.R, d.B, d.I, d.H), optional=d.B == 0),
        _ptr(gu_save, "gu_save", bf, (M, 2 * d.I), optional=True),
        _ptr(act, "act", bf, (M, d.I)),
        _ptr(y, "y", bf, (M, d.H)),
    )
    _check(_lib().moonep_grouped_ffn(ctypes.byref(d), *args, _stream(stream)), "moonep_grouped_ffn")


def moonep_grouped_ffn_backward(d: Dims, plan_ws, cu_seqlens, recv, gu_save, act, dy, w13_home,
                                w2_home, w13_slot, w2_slot, drecv, dw13_home, dw2_home, dw13_red,
                                dw2_red, stream=None) -> None:
    """gu_save holds Gt|U from the forward on entry and dGt|dU on return."""
    torch = _torch()
    bf, f32 = torch.bfloat16, torch.float32
    M = d.R * d.S * d.K
    nb = d.B == 0
    args = (
        _ws(d, plan_ws),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (d.R, d.E + d.B + 1)),
        _ptr(recv, "recv", bf, (M, d.H)),
        _ptr(gu_save, "gu_save", bf, (M, 2 * d.I)),
        _ptr(act, "act", bf, (M, d.I)),
        _ptr(dy, "dy", bf, (M, d.H)),
        _ptr(w13_home, "w13_home", bf, (d.E, d.H, 2 * d.I)),
        _ptr(w2_home, "w2_home", bf, (d.E, d.I, d.H)),
        _ptr(w13_slot, "w13_slot", bf, (d.R, d.B, d.H, 2 * d.I), optional=nb),
        _ptr(w2_slot, "w2_slot", bf, (d.R, d.B, d.I, d.H), optional=nb),
        _ptr(drecv, "drecv", bf, (M, d.H)),
        _ptr(dw13_home, "dw13_home", f32, (d.E, d.H, 2 * d.I)),
        _ptr(dw2_home, "dw2_home", f32, (d.E, d.I, d.H)),
        _ptr(dw13_red, "dw13_red", f32, (d.R, d.B, d.H, 2 * d.I), optional=nb),
        _ptr(dw2_red, "dw2_red", f32, (d.R, d.B, d.I, d.H), optional=nb),
    )
    _check(_lib().moonep_grouped_ffn_backward(ctypes.byref(d), *args, _stream(stream)),
           "moonep_grouped_ffn_backward")


def moonep_reduce_grad(d: Dims, plan_ws, dw13_home, dw2_home, dw13_red, dw2_red, stream=None) -> None:
    torch = _torch()
    f32 = torch.float32
    nb = d.B == 0
    args = (
        _ws(d, plan_ws),
        _ptr(dw13_home, "dw13_home", f32, (d.E, d.H, 2 * d.I)),
        _ptr(dw2_home, "dw2_home", f32, (d.E, d.I, d.H)),
        _ptr(dw13_red, "dw13_red", f32, (d.R, d.B, d.H, 2 * d.I), optional=nb),
        _ptr(dw2_red, "dw2_red", f32, (d.R, d.B, d.I, d.H), optional=nb),
    )
    _check(_lib().moonep_reduce_grad(ctypes.byref(d), *args, _stream(stream)), "moonep_reduce_grad")
