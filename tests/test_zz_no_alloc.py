"""The allocation-free planning entry point against moonep_plan.

moonep_plan_noalloc keeps its plan workspace in a static device array of the library.  Two calls
in a row, the second on a smaller problem (so stale workspace contents from the first call are
there to be misread), must give cu_seqlens, dest and stats bit-identical to moonep_plan, which
are in turn the oracle's; and dims whose workspace exceeds the static array are refused on the
host.  Every call goes through the C ABI (ctypes)."""
import ctypes

import numpy as np
import pytest
import torch

import balanced_token_dispatch_moonep_amd as M
import oracle as O
import workload as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _plan_both(cfg, B, training):
    topk, _, _ = W.routing_for(cfg)
    d = M.Dims.make(cfg.R, cfg.E, B, cfg.S, cfg.K, cfg.H, training=training)
    tk = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).to(DEV)
    outs = []
    for noalloc in (False, True):
        cu = torch.full((d.R, d.E + d.B + 1), -7, dtype=torch.int32, device=DEV)
        dest = torch.full((d.R, d.S, d.K), -7, dtype=torch.int32, device=DEV)
        st = torch.full((M.NSTATS,), -7, dtype=torch.int32, device=DEV)
        if noalloc:
            M.moonep_plan_noalloc(d, tk, cu, dest, st)
        else:
            ws = torch.empty(M.moonep_plan_workspace_bytes(d), dtype=torch.uint8, device=DEV)
            M.moonep_plan(d, tk, ws, cu, dest, st)
        torch.cuda.synchronize()
        outs.append((cu.cpu().numpy(), dest.cpu().numpy(), st.cpu().numpy()))
    return topk, outs


@pytest.mark.parametrize("first,second", [
    # the full plan + dispatch + combine shape, then a small skewed one (fallback at B = 0)
    (dict(name="skew", maxvio=8.0, B=4, training=False), dict(name="tiny", lam=2.0, B=0, training=True)),
    (dict(name="skew", maxvio=4.0, B=3, training=False), dict(name="skew", S=640, maxvio=2.0, B=2,
                                                             training=False)),
])
def test_noalloc_matches_plan_twice(first, second):
    for spec in (first, second):
        spec = dict(spec)
        cfg = W.CONFIGS[spec.pop("name")].with_(**{k: v for k, v in spec.items() if k not in ("B", "training")})
        print("noalloc plan", cfg, spec["B"], flush=True)
        topk, (ref, got) = _plan_both(cfg, spec["B"], spec["training"])
        for a, b in zip(ref, got):
            np.testing.assert_array_equal(a, b)
        plan = O.make_plan(topk, cfg.E, spec["B"], training=spec["training"])
        np.testing.assert_array_equal(got[0], plan.cu)
        np.testing.assert_array_equal(got[1], O.destinations(topk, plan))


def test_noalloc_rejects_oversized_dims():
    d = M.Dims.make(R=16, E=1024, B=4, S=65536, K=8, H=128)
    assert M.moonep_plan_workspace_bytes(d) > M.NOALLOC_WS_BYTES
    g = ctypes.c_void_p(0x10000)
    assert M.lib.moonep_plan_noalloc(ctypes.byref(d), g, g, g, g, None) == -5
