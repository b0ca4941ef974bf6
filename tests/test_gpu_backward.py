"""GPU parity of the backward pass (kdn_backward, through the C ABI) against
the fp64 oracle's adjoint (itself pinned by finite differences) on identical
seeded inputs and cotangents.  Tolerance as the forward: max relative error
per gradient tensor 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (the
arithmetic is fp32 in both cases)."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import TOKEN_INPUTS, check_dc0, rel_err, sample_pairs, to_dev, tol

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0")


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _f32dev(a, dev):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)


def run_backward(dev, w, x, ct, st):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dO = torch.from_numpy(ct["dO"]).to(tdt).to(dev)
    g = kdn.backward(**t, mu=w.mu, dO=dO, dS_T=_f32dev(ct["dS_T"], dev), dp_T=_f32dev(ct["dp_T"], dev),
                     variant=w.variant, S0=_f32dev(st["S0"], dev), p0=_f32dev(st["p0"], dev))
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in g.items()}


def oracle_backward(w, x, ct, st):
    return oracle.backward(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, dO=ct["dO"],
                           dS_T=ct["dS_T"], dp_T=ct["dp_T"], S0=st["S0"], p0=st["p0"], variant=w.variant)


def check(name, got, ref, dtype, keys=GRADS + ("dc0",)):
    errs = {k: rel_err(got[k], ref[k]) for k in keys}
    print(f"{name}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        if k != "dc0":  # dc0 = the sum of dp0: checked against the kernel's own dp0
            assert e <= tol(dtype), (name, k, e)
    if "dc0" in keys:
        check_dc0(got["dc0"], got["dp0"])


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 31, 32, 33, 100])
def test_backward_small(dev, variant, dtype, dk, dv, T):
    # strong process noise so that gains and their derivatives are large
    w = wl.Workload("bwd", variant, dtype, 2, T, 2, dk, dv, float(dk), "uniform", 100 + T, omega_loc=0.0)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)
    st = {"S0": None, "p0": None}
    got = run_backward(dev, w, x, ct, st)
    ref = oracle_backward(w, x, ct, st)
    check(f"{variant}/{dtype}/dk{dk}/dv{dv}/T{T}", got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 33, 100])
def test_backward_grouped_noise(dev, dtype, dk, dv, T):
    w = wl.Workload("bwd_grp", "grouped", dtype, 2, T, 2, dk, dv, float(dk), "uniform", 400 + T, omega_loc=0.0,
                    rgroups=dv // 64)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)
    st = wl.decode_state(w) if T == 33 else {"S0": None, "p0": None}
    got = run_backward(dev, w, x, ct, st)
    ref = oracle_backward(w, x, ct, st)
    check(f"grouped/{dtype}/dk{dk}/dv{dv}/T{T}", got, ref, dtype)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_backward_with_initial_state_and_config_distributions(dev, variant):
    w = wl.Workload("bwd_state", variant, "bf16", 3, 77, 2, 128, 128, 128.0, "uniform", 7)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)
    st = wl.decode_state(w)
    got = run_backward(dev, w, x, ct, st)
    ref = oracle_backward(w, x, ct, st)
    check(f"{variant} with S0/p0", got, ref, "bf16")


def test_backward_output_cotangent_only(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("bwd_o", "diagonal", "f32", 2, 45, 2, 64, 64, 64.0, "one", 8)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=False)
    t = to_dev(x, "f32", dev)
    g = kdn.backward(**t, mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(dev))
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in g.items()}
    ref = oracle.backward(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, dO=ct["dO"])
    check("dO only", got, ref, "f32")


def test_backward_empty_sequence_passes_state_cotangents_through(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("bwd_empty", "diagonal", "bf16", 2, 0, 3, 128, 128, 128.0, "uniform", 9)
    x = wl.forward_inputs(w)
    t = to_dev(x, "bf16", dev)
    gen = torch.Generator(device="cpu").manual_seed(9)
    dS_T = torch.randn(2, 3, 128, 128, generator=gen).to(dev)
    dp_T = torch.randn(2, 3, 128, generator=gen).to(dev)
    g = kdn.backward(**t, mu=w.mu, dS_T=dS_T, dp_T=dp_T)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS_T) and torch.equal(g["dp0"], dp_T)
    # dc0 sums 256 fp32 values per head in the kernel's order, the reference
    # in torch's: the orders differ by a few ulps of the partial sums (|x| <~ 4)
    assert torch.allclose(g["dc0"], dp_T.sum(dim=(0, 2)), rtol=1e-5, atol=1e-4)


def test_backward_deterministic(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("bwd_det", "diagonal", "bf16", 2, 70, 4, 128, 128, 128.0, "uniform", 10)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w)
    t = to_dev(x, "bf16", dev)
    dO = torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev)
    a = kdn.backward(**t, mu=w.mu, dO=dO)
    b = kdn.backward(**t, mu=w.mu, dO=dO)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_backward_chunked_segments(dev, dk, dv):
    # the diagonal bf16 backward runs in chunk form: T = 1100 is 34 full
    # chunks and a 12-token tail, and three segments (512, 512, 76 tokens)
    # of the uncertainty adjoint, whose maps carry dp across them
    w = wl.Workload("bwd_seg", "diagonal", "bf16", 1, 1100, 2, dk, dv, float(dk), "uniform", 120 + dk + dv,
                    omega_loc=-1.0)
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)
    rng = np.random.default_rng(121)
    st = {"S0": wl.round_bf16(rng.standard_normal((1, 2, dk, dv)).astype(np.float32) * 0.2),
          "p0": rng.uniform(0.5, 2.0, (1, 2, dk)).astype(np.float32)}
    got = run_backward(dev, w, x, ct, st)
    ref = oracle_backward(w, x, ct, st)
    check(f"chunked/segments/dk{dk}/dv{dv}", got, ref, "bf16")


def test_backward_chunked_with_a_pair_out_of_range(dev):
    # one (batch, head) pair has a chunk of alpha = 1e-6, outside the chunked
    # form's range: that pair takes the token recurrence's adjoint, the
    # others the chunked one, in the same call
    w = wl.Workload("bwd_mix", "diagonal", "bf16", 2, 300, 2, 128, 128, 128.0, "uniform", 130, omega_loc=-1.0)
    x = wl.forward_inputs(w)
    x["alpha"][1, 96:128, 0] = wl.round_bf16(np.full((32, 128), 1e-6, np.float32))
    ct = wl.backward_cotangents(w, with_state=True)
    st = {"S0": None, "p0": None}
    got = run_backward(dev, w, x, ct, st)
    ref = oracle_backward(w, x, ct, st)
    check("chunked/mixed range", got, ref, "bf16")


@pytest.mark.parametrize("name", ["diag_bf16_b8_t4096_h16_d128", "iso_bf16_b8_t4096_h16_d128"])
def test_backward_full_size_sampled_heads(dev, name):
    """The B=8, T=4096, H=16, d=128 workloads (the diagonal one in the launch
    configuration the benchmark times); the oracle runs on sampled heads."""
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.WORKLOADS[name]
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=False)
    t = to_dev(x, "bf16", dev)
    g = kdn.backward(**t, mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev), variant=w.variant)
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in g.items()}
    pairs = sample_pairs(w.B, w.H, 2, seed=w.seed)
    worst = {k: 0.0 for k in GRADS}
    for b, h in pairs:
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in TOKEN_INPUTS}
        ref = oracle.backward(**sub, c0=x["c0"][h:h + 1], mu=w.mu,
                              dO=np.ascontiguousarray(ct["dO"][b:b + 1, :, h:h + 1]), variant=w.variant)
        for k in GRADS:
            gk = got[k][b:b + 1, :, h:h + 1] if k not in ("dS0", "dp0") else got[k][b:b + 1, h:h + 1]
            worst[k] = max(worst[k], rel_err(gk, ref[k]))
    print(f"full size {name} pairs={pairs}: " + " ".join(f"{k}={v:.1e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (k, e)
    for k in GRADS:
        assert np.all(np.isfinite(got[k])), k


def test_backward_full_size_every_pair(dev):
    """The diagonal bf16 backward at B=8, T=4096, H=16, d=128 on its smallest
    workspace (the benchmark's configuration: eight 512-token slabs), every
    (batch, head) pair against oracle.backward; reports the worst pair."""
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.WORKLOADS["diag_bf16_b8_t4096_h16_d128"]
    x = wl.forward_inputs(w)
    ct = wl.backward_cotangents(w, with_state=False)
    t = to_dev(x, "bf16", dev)
    ws = torch.empty(kdn.backward_workspace_size(w.B, w.T, w.H, w.dk, w.dv, w.variant, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    g = kdn.backward(**t, mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev), variant=w.variant,
                     workspace=ws)
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in g.items()}
    del g, ws, t
    ref = oracle.backward(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, dO=ct["dO"], variant=w.variant)
    errs = {k: rel_err(got[k], ref[k]) for k in GRADS}
    worst = {}
    for k in GRADS:
        per = [rel_err(got[k][b, :, h] if k not in ("dS0", "dp0") else got[k][b, h],
                       ref[k][b, :, h] if k not in ("dS0", "dp0") else ref[k][b, h])
               for b in range(w.B) for h in range(w.H)]
        j = int(np.argmax(per))
        worst[k] = (per[j], divmod(j, w.H))
    print("backward full size, every pair: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    print("worst pair: " + " ".join(f"{k}={v[0]:.2e}{v[1]}" for k, v in worst.items()), flush=True)
    for k in GRADS:
        assert np.all(np.isfinite(got[k])), k
        assert errs[k] <= tol("bf16"), (k, errs[k])
        assert worst[k][0] <= tol("bf16"), (k, worst[k])
