"""kdn_backward_noalloc (the backward with the library's static device scratch
in place of a workspace) against kdn_backward with a caller workspace, through
the C ABI: two calls in a row, the second smaller, each bit-identical to the
workspace form (same kernels), and sizes beyond the scratch refused."""
import ctypes

import numpy as np
import pytest

from kalman_delta_network_amd import workloads as wl

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0", "dc0")


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _case(w, dev):
    import torch
    x = wl.forward_inputs(w)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev)
         for n in ("q", "k", "v", "alpha", "omega", "r")}
    t["c0"] = torch.from_numpy(x["c0"]).to(dev)
    ct = wl.backward_cotangents(w)
    cot = {"dO": torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev),
           "dS_T": torch.from_numpy(ct["dS_T"]).to(dev), "dp_T": torch.from_numpy(ct["dp_T"]).to(dev)}
    return t, cot


def _outputs(w, dev, fill):
    import torch
    shp = {"dq": (w.B, w.T, w.H, w.dk), "dk": (w.B, w.T, w.H, w.dk), "dv": (w.B, w.T, w.H, w.dv),
           "dalpha": (w.B, w.T, w.H, w.dk), "domega": (w.B, w.T, w.H, w.dk), "dr": (w.B, w.T, w.H),
           "dS0": (w.B, w.H, w.dk, w.dv), "dp0": (w.B, w.H, w.dk), "dc0": (w.H,)}
    return {n: torch.full(s, fill, dtype=torch.float32, device=dev) for n, s in shp.items()}


def _call_noalloc(lib, w, t, cot, g, stream):
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    return lib.kdn_backward_noalloc(p(t["q"]), p(t["k"]), p(t["v"]), p(t["alpha"]), p(t["omega"]), p(t["r"]),
                                    p(t["c0"]), ctypes.c_float(w.mu), 0, 1, w.B, w.T, w.H, w.dk, w.dv, None, None,
                                    p(cot["dO"]), p(cot["dS_T"]), p(cot["dp_T"]), *(p(g[n]) for n in GRADS),
                                    ctypes.c_void_p(stream))


def test_noalloc_matches_workspace_backward_twice(dev):
    import torch
    import kalman_delta_network_amd as kdn
    lib = kdn.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    cases = [wl.Workload("noalloc1", "diagonal", "bf16", 2, 300, 3, 128, 128, 128.0, "uniform", 3101, omega_loc=-1.0),
             wl.Workload("noalloc2", "diagonal", "bf16", 1, 70, 2, 64, 128, 64.0, "uniform", 3102, omega_loc=-1.0)]
    for w in cases:  # the second call is smaller: the scratch keeps the first call's contents
        t, cot = _case(w, dev)
        g = _outputs(w, dev, float("nan"))
        st = _call_noalloc(lib, w, t, cot, g, stream)
        assert st == 0, (st, lib.kdn_last_error())
        ref = kdn.backward(**t, mu=w.mu, **cot)
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(g[n], ref[n]), (w.name, n)
        print(f"{w.name}: bit-identical to kdn_backward", flush=True)


def test_noalloc_refuses_sizes_beyond_the_scratch(dev):
    import torch
    import kalman_delta_network_amd as kdn
    lib = kdn.load_library()
    w = wl.Workload("noalloc_big", "diagonal", "bf16", 1, 8192, 16, 128, 128, 128.0, "uniform", 3103)
    assert kdn.backward_workspace_size(w.B, w.T, w.H, w.dk, w.dv, "diagonal", torch.bfloat16) > \
        kdn.NOALLOC_SCRATCH_BYTES
    t, cot = _case(w, dev)
    g = _outputs(w, dev, 7.0)
    st = _call_noalloc(lib, w, t, cot, g, torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    assert st == kdn.KDN_ERR_WORKSPACE, st
    assert b"static" in lib.kdn_last_error()
    for n in GRADS:
        assert bool(torch.all(g[n] == 7.0)), n  # nothing was written
