"""C-ABI checks that need no GPU: the library loads, exports every function that
include/moonep.h declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import balanced_token_dispatch_moonep_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moonep.h")

EINVAL, EALIGN, EHIP, ENOTSUP = -1, -2, -3, -4


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moonep_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = M.lib
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(M.EXPORTED)


def test_version_and_strerror():
    assert "gfx950" in M.moonep_version()
    for code in (0, EINVAL, EALIGN, EHIP, ENOTSUP, -99):
        assert isinstance(M.moonep_strerror(code), str)


def _dims(**kw):
    base = dict(R=8, E=256, B=4, S=4096, K=8, H=7168, I=2048)
    base.update(kw)
    return M.Dims.make(**base)


def test_workspace_bytes_pure_host():
    n = M.moonep_plan_workspace_bytes(_dims())
    assert 1 << 20 < n < 64 << 20
    # grows with the number of chunks
    assert M.moonep_plan_workspace_bytes(_dims(S=8192)) > n
    lib = M.lib
    for bad in (_dims(E=250), _dims(R=0), _dims(K=0), _dims(K=17), _dims(H=7), _dims(B=-1),
                _dims(R=2, E=256)):                        # E/R = 128 > 64 home experts per rank
        assert lib.moonep_plan_workspace_bytes(ctypes.byref(bad)) == 0


VP = ctypes.c_void_p


def test_plan_rejects_null_and_misaligned():
    lib = M.lib
    d = _dims()
    good = VP(0x10000)
    assert lib.moonep_plan(None, good, good, good, good, good, None) == EINVAL
    assert lib.moonep_plan(ctypes.byref(d), None, good, good, good, good, None) == EINVAL
    assert lib.moonep_plan(ctypes.byref(d), good, good, good, None, good, None) == EINVAL
    assert lib.moonep_plan(ctypes.byref(d), VP(0x10004), good, good, good, good, None) == EALIGN
    bad = _dims(E=255)
    assert lib.moonep_plan(ctypes.byref(bad), good, good, good, good, good, None) == EINVAL
    bad = _dims()
    bad.flags = 1024          # no such flag
    assert lib.moonep_plan(ctypes.byref(bad), good, good, good, good, good, None) == EINVAL


def test_dispatch_combine_reject():
    lib = M.lib
    d = _dims()
    g = VP(0x10000)
    assert lib.moonep_dispatch(ctypes.byref(d), None, g, None, g, None) == EINVAL
    assert lib.moonep_dispatch(ctypes.byref(d), g, VP(0x10002), None, g, None) == EALIGN
    assert lib.moonep_dispatch(ctypes.byref(d), g, g, VP(0x10008), g, None) == EALIGN
    assert lib.moonep_combine(ctypes.byref(d), g, g, None, None, None) == EINVAL
    assert lib.moonep_combine(ctypes.byref(_dims(H=12)), g, g, None, g, None) == EINVAL


def test_ffn_rejects_unsupported():
    lib = M.lib
    g = VP(0x10000)
    args = [g] * 10 + [None]
    # the expert GEMM is bf16-only and needs H, I multiples of 64
    assert lib.moonep_grouped_ffn(ctypes.byref(_dims(f32_rows=True)), *args) == ENOTSUP
    assert lib.moonep_grouped_ffn(ctypes.byref(_dims(H=7176)), *args) == ENOTSUP
    assert lib.moonep_grouped_ffn(ctypes.byref(_dims(I=2056)), *args) == ENOTSUP
    assert lib.moonep_grouped_ffn(ctypes.byref(_dims(I=0)), *args) == EINVAL
    args2 = [g, g, None] + [g] * 8 + [None]
    assert lib.moonep_grouped_ffn(ctypes.byref(_dims()), *args2) == EINVAL
    bargs = [g] * 16 + [None]
    bargs[3] = None          # gu_save is required by the backward
    assert lib.moonep_grouped_ffn_backward(ctypes.byref(_dims()), *bargs) == EINVAL
    bargs[3] = VP(0x10001)
    assert lib.moonep_grouped_ffn_backward(ctypes.byref(_dims()), *bargs) == EALIGN


def test_prefetch_reduce_reject():
    lib = M.lib
    g = VP(0x10000)
    assert lib.moonep_prefetch(ctypes.byref(_dims()), None, g, g, g, g, None) == EINVAL
    assert lib.moonep_prefetch(ctypes.byref(_dims()), g, g, g, None, g, None) == EINVAL
    assert lib.moonep_reduce_grad(ctypes.byref(_dims()), g, g, g, g, VP(0x1000c), None) == EALIGN
    assert lib.moonep_reduce_grad(ctypes.byref(_dims(I=0)), g, g, g, g, g, None) == EINVAL


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    d = M.Dims.make(R=2, E=4, B=1, S=64, K=2, H=64)
    t = torch.zeros((2, 64, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        M.moonep_plan(d, t, t, t, t, t, stream=0)


def test_flag_constants_match_header():
    """The binding's flag and phase constants are the header's #define values."""
    text = open(HEADER).read()
    found = dict((k, int(v)) for k, v in re.findall(r"#define MOONEP_([A-Z0-9_]+) (\d+)u", text))
    expect = {"TRAINING": M.TRAINING, "F32_ROWS": M.F32_ROWS, "GRAD_ACCUM": M.GRAD_ACCUM,
              "PHASE_GATE_UP": M.PHASE_GATE_UP, "PHASE_DOWN": M.PHASE_DOWN, "PHASE_DACT": M.PHASE_DACT,
              "PHASE_DX": M.PHASE_DX, "PHASE_DW2": M.PHASE_DW2, "PHASE_DW13": M.PHASE_DW13}
    for k, v in expect.items():
        assert found[k] == v, k
    bits = [v for k, v in expect.items()]
    assert len(set(bits)) == len(bits) and all(b & (b - 1) == 0 for b in bits)


def test_pool_bytes_match_memory_contract():
    """One rank's pooled slot and reduce buffers are the memory contract's prefetch and fp32
    reduce buffers (pinned to the thakicloud.com post's Table 2 through the oracle), and
    pooling keeps them constant in depth."""
    import oracle as O
    from balanced_token_dispatch_moonep_amd.layer import MoonEPPool, stack_slot_bytes
    for B, training in ((4, False), (32, True)):
        got = MoonEPPool.nbytes(1, B, 7168, 2048, training)
        ref = O.buffer_bytes(B, 4096, 8, 7168, 2048, training=training)
        assert got["prefetch"] == ref["prefetch"] and got["reduce"] == ref["reduce"]
    one = stack_slot_bytes(8, 4, 7168, 2048, 1, pooled=True, training=True)
    assert stack_slot_bytes(8, 4, 7168, 2048, 61, pooled=True, training=True) == one
    assert stack_slot_bytes(8, 4, 7168, 2048, 61, pooled=False, training=True) == 61 * one
