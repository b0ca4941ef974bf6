"""GPU parity over the whole decay range 0 < alpha <= 1 (through the C ABI,
against the fp64 oracle, 2e-2 for bf16 inputs with fp32 state).

The chunked kernel references in-chunk decays to the chunk's midpoint, so it
covers half-chunk decays down to 2^-96 (alpha ~ sigmoid(N(-3, 0.5)) is well
inside); a chunk below that switches its workgroup to the token recurrence
from that chunk on.  These cases exercise both: strong decay everywhere, and
full chunks at alpha = 1e-3 and 1e-6 in the middle or at the tail of the
sequence, for every variant, both chunk widths, the gated forms, grouped
observation noise and packed batches."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_forward, TOKEN_INPUTS, oracle_forward, p_rel_err, rel_err, to_dev, tol

pytestmark = pytest.mark.gpu

L = 32  # tokens per chunk of the chunked kernel


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def set_alpha(x, variant, lo, hi, value, gated=False):
    """alpha (or its pre-activation) = value on tokens [lo, hi) of every
    sequence and head (bf16-rounded, as the workloads are)."""
    name = "z_alpha" if gated else "alpha"
    v = np.log(value / (1.0 - value)) if gated else value
    x[name][:, lo:hi] = wl.round_bf16(np.full(x[name][:, lo:hi].shape, v, np.float32))


def check(name, got, ref):
    return check_forward(name, got, ref, "bf16")


def run(dev, w, x, algo, gated=False):
    import torch
    import kalman_delta_network_amd as kdn
    if gated:
        names = ("q", "k", "v", "z_alpha", "z_omega", "z_r")
        t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev) for n in names}
        t["c0"] = torch.from_numpy(x["c0"]).to(dev)
        o, S, p = kdn.forward_gated(**t, mu=w.mu, variant=w.variant, algo=algo)
    else:
        o, S, p = kdn.forward(**to_dev(x, "bf16", dev), mu=w.mu, variant=w.variant, algo=algo)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


CASES = [
    # name, alpha_loc, (first chunk, last chunk + 1, value) or None, T
    ("strong", -3.0, None, 160),
    ("chunk_1e-3", 2.0, (2, 3, 1e-3), 160),
    ("chunk_1e-6", 2.0, (1, 2, 1e-6), 160),
    ("tail_1e-6", 2.0, (4, 5, 1e-6), 150),
    ("first_1e-3", 2.0, (0, 1, 1e-3), 100),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("algo", ["chunked_wide", "chunked_narrow", "recurrent"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_alpha_range(dev, case, algo, variant, dk, dv):
    name, aloc, chunk, T = case
    w = wl.Workload("arange", variant, "bf16", 2, T, 2, dk, dv, float(dk), "uniform", 2100 + T + dk,
                    alpha_loc=aloc, omega_loc=-2.0)
    x = wl.forward_inputs(w)
    if chunk:
        set_alpha(x, variant, chunk[0] * L, min(T, chunk[1] * L), chunk[2])
    check(f"{name}/{variant}/{algo}/dk{dk}", run(dev, w, x, algo), oracle_forward(w, x))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("algo", ["chunked_wide", "chunked_narrow"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_alpha_range_gated(dev, case, algo, variant):
    name, aloc, chunk, T = case
    w = wl.Workload("arange_g", variant, "bf16", 2, T, 2, 128, 128, 128.0, "uniform", 2200 + T,
                    alpha_loc=aloc, omega_loc=-2.0)
    x = wl.gated_inputs(w)
    if chunk:
        set_alpha(x, variant, chunk[0] * L, min(T, chunk[1] * L), chunk[2], gated=True)
    ref = oracle.forward_gated(**{n: x[n] for n in ("q", "k", "v", "z_alpha", "z_omega", "z_r")}, c0=x["c0"],
                               mu=w.mu, variant=variant)
    check(f"gated/{name}/{variant}/{algo}", run(dev, w, x, algo, gated=True), ref)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_alpha_range_grouped(dev, case):
    import torch
    import kalman_delta_network_amd as kdn
    name, aloc, chunk, T = case
    w = wl.Workload("arange_gr", "grouped", "bf16", 2, T, 2, 128, 128, 128.0, "uniform", 2300 + T,
                    alpha_loc=aloc, omega_loc=-2.0, rgroups=2)
    x = wl.forward_inputs(w)
    if chunk:
        set_alpha(x, "grouped", chunk[0] * L, min(T, chunk[1] * L), chunk[2])
    o, S, p = kdn.forward(**to_dev(x, "bf16", dev), mu=w.mu, variant="grouped", algo="chunked")
    torch.cuda.synchronize()
    ref = oracle.forward_grouped(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu)
    check(f"grouped/{name}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_alpha_range_packed(dev, variant):
    # one sequence has a chunk at alpha = 1e-6, the others are ordinary
    import torch
    import kalman_delta_network_amd as kdn
    lengths = [70, 0, 130, 33]
    w = wl.Workload("arange_var", variant, "bf16", len(lengths), 0, 2, 128, 128, 128.0, "uniform", 2400,
                    omega_loc=-2.0)
    x = wl.varlen_inputs(w, lengths)
    cu = x["cu_seqlens"]
    lo = int(cu[2]) + 32  # the second chunk of the third sequence
    x["alpha"][lo:lo + 32] = wl.round_bf16(np.full(x["alpha"][lo:lo + 32].shape, 1e-6, np.float32))
    t = to_dev(x, "bf16", dev)
    o, S, p = kdn.forward_varlen(**t, cu_seqlens=torch.from_numpy(cu).to(dev), mu=w.mu, variant=variant,
                                 algo="chunked", order=torch.from_numpy(kdn.longest_first(cu)).to(dev))
    torch.cuda.synchronize()
    ref = oracle.forward_varlen(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, cu_seqlens=cu,
                                variant=variant)
    check(f"packed/{variant}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref)


def test_fallback_continues_in_place(dev):
    # S_T is the S0 buffer (continuation in place) and the sequence leaves the
    # chunked form's range: the hand-off starts from the carried state, not S0
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("arange_inpl", "diagonal", "bf16", 2, 130, 2, 128, 128, 128.0, "uniform", 2500, omega_loc=-1.0)
    x = wl.forward_inputs(w)
    set_alpha(x, "diagonal", 64, 96, 1e-6)
    st = wl.decode_state(w)
    t = to_dev(x, "bf16", dev)
    S0 = torch.from_numpy(st["S0"]).to(dev)
    p0 = torch.from_numpy(st["p0"]).to(dev)
    o = torch.empty((2, 130, 2, 128), dtype=torch.bfloat16, device=dev)
    pT = torch.empty_like(p0)
    kdn.forward(**t, mu=w.mu, S0=S0, p0=p0, algo="chunked", out=(o, S0, pT))
    torch.cuda.synchronize()
    ref = oracle_forward(w, x, S0=st["S0"], p0=st["p0"])
    check("in_place", (o.float().cpu().numpy(), S0.cpu().numpy(), pT.cpu().numpy()), ref)
