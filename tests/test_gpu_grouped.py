"""GPU parity of the diagonal variant with grouped observation noise (one r
and one uncertainty state per group of 64 value columns; "Memory by Design:
Probabilistic Sequence Layers", per-column and grouped observation noise)
against oracle.forward_grouped, through the C ABI.  Tolerance as the other
forward tests."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_forward, TOKEN_INPUTS, rel_err, sample_pairs, to_dev, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _f32(a, dev):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def run(dev, w, x, algo, S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    o, S, p = kdn.forward(**t, mu=w.mu, variant="grouped", S0=_f32(S0, dev), p0=_f32(p0, dev), algo=algo)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


def check(name, got, ref, dtype):
    return check_forward(name, got, ref, dtype)


@pytest.mark.parametrize("algo,dtype", [("recurrent", "f32"), ("recurrent", "bf16"), ("chunked", "bf16")])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 33, 100])
def test_grouped_forward_small(dev, algo, dtype, dk, dv, T):
    w = wl.Workload("grp", "grouped", dtype, 2, T, 3, dk, dv, float(dk), "uniform", 300 + T, omega_loc=-1.0,
                    rgroups=dv // 64)
    x = wl.forward_inputs(w)
    got = run(dev, w, x, algo)
    ref = oracle.forward_grouped(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu)
    check(f"{algo}/{dtype}/dk{dk}/dv{dv}/T{T}", got, ref, dtype)


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_grouped_forward_with_initial_state(dev, algo):
    w = wl.Workload("grp_s", "grouped", "bf16", 2, 70, 2, 128, 128, 128.0, "uniform", 31, rgroups=2)
    x = wl.forward_inputs(w)
    st = wl.decode_state(w)
    got = run(dev, w, x, algo, st["S0"], st["p0"])
    ref = oracle.forward_grouped(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, S0=st["S0"], p0=st["p0"])
    check(f"{algo} with S0/p0", got, ref, "bf16")


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_grouped_with_equal_groups_is_the_diagonal_kernel_bit_for_bit(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("grp_eq", "grouped", "bf16", 2, 77, 2, 128, 128, 128.0, "uniform", 32, rgroups=2)
    x = wl.forward_inputs(w)
    x["r"][..., 1] = x["r"][..., 0]
    t = to_dev(x, "bf16", dev)
    og, Sg, pg = kdn.forward(**t, mu=w.mu, variant="grouped", algo=algo)
    td = dict(t, r=t["r"][..., 0].contiguous())
    od, Sd, pd = kdn.forward(**td, mu=w.mu, variant="diagonal", algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(og, od) and torch.equal(Sg, Sd)
    assert torch.equal(pg[:, :, 0], pd) and torch.equal(pg[:, :, 1], pd)


def test_grouped_decode_steps(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("grp_dec", "grouped", "bf16", 6, 1, 4, 128, 128, 128.0, "uniform", 33, rgroups=2)
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    Sr, pr = st["S0"].astype(np.float64), st["p0"].astype(np.float64)
    for s in range(5):
        x = wl.decode_tokens(w, s)
        o = kdn.step(**to_dev(x, "bf16", dev), mu=w.mu, S=S, p=p, variant="grouped")
        ref = oracle.forward_grouped(**{n: x[n][:, None] for n in TOKEN_INPUTS}, c0=np.ones(w.H, np.float32),
                                     mu=w.mu, S0=Sr, p0=pr)
        Sr, pr = ref["S"], ref["p"]
    torch.cuda.synchronize()
    check("decode", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()),
          {"o": ref["o"][:, 0], "S": Sr, "p": pr}, "bf16")


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_grouped_varlen(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("grp_var", "grouped", "bf16", 4, 0, 2, 128, 128, 128.0, "uniform", 34, rgroups=2)
    x = wl.varlen_inputs(w, [33, 0, 1, 70])
    t = to_dev(x, "bf16", dev)
    o, S, p = kdn.forward_varlen(**t, cu_seqlens=torch.from_numpy(x["cu_seqlens"]).to(dev), mu=w.mu,
                                 variant="grouped", algo=algo)
    torch.cuda.synchronize()
    ref = oracle.forward_varlen(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, cu_seqlens=x["cu_seqlens"],
                                variant="grouped")
    check(f"varlen/{algo}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref, "bf16")


def test_grouped_full_size_sampled_heads(dev):
    w = wl.WORKLOADS["grouped_bf16_b8_t4096_h16_d128"]
    x = wl.forward_inputs(w)
    o, S, p = run(dev, w, x, "auto")
    worst = {"o": 0.0, "S": 0.0, "p": 0.0}
    for b, h in sample_pairs(w.B, w.H, 3, seed=w.seed):
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in TOKEN_INPUTS}
        ref = oracle.forward_grouped(**sub, c0=x["c0"][h:h + 1], mu=w.mu)
        for key, g in (("o", o[b:b + 1, :, h:h + 1]), ("S", S[b:b + 1, h:h + 1]), ("p", p[b:b + 1, h:h + 1])):
            worst[key] = max(worst[key], rel_err(g, ref[key]))
    print("grouped full size: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (k, e)
