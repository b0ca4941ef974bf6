"""GPU parity of the gated backward (kdn_backward_gated: gradients of the
gated forward, the gate pre-activations included) against
oracle.backward_gated (pinned by finite differences of oracle.forward_gated)
on identical seeded inputs and cotangents, through the C ABI.  Tolerance:
max relative error per gradient tensor 1e-4 (fp32 inputs) or 2e-2 (bf16
inputs)."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_dc0, rel_err, tol

pytestmark = pytest.mark.gpu

GATED = ("q", "k", "v", "z_alpha", "z_omega", "z_r")
GRADS = ("dq", "dk", "dv", "dz_alpha", "dz_omega", "dz_r", "dS0", "dp0", "dc0")


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


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 33, 100])
@pytest.mark.parametrize("with_state", [False, True])
def test_gated_backward(dev, variant, dtype, dk, dv, T, with_state):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gbwd", variant, dtype, 2, T, 2, dk, dv, float(dk), "uniform", 1700 + T + dk, omega_loc=0.0)
    x = wl.gated_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)
    st = wl.decode_state(w) if with_state else {"S0": None, "p0": None}
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(tdt).to(dev) for n in GATED}
    g = kdn.backward_gated(**t, c0=_f32(x["c0"], dev), mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(tdt).to(dev),
                           dS_T=_f32(ct["dS_T"], dev), dp_T=_f32(ct["dp_T"], dev), variant=variant,
                           S0=_f32(st["S0"], dev), p0=_f32(st["p0"], dev))
    torch.cuda.synchronize()
    ref = oracle.backward_gated(**{n: x[n] for n in GATED}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                                dp_T=ct["dp_T"], S0=st["S0"], p0=st["p0"], variant=variant)
    errs = {k: rel_err(g[k].cpu().numpy(), ref[k]) for k in GRADS}
    print(f"gated bwd {variant}/{dtype}/dk{dk}/dv{dv}/T{T}/state{int(with_state)}: "
          + " ".join(f"{k}={e:.1e}" for k, e in errs.items()), flush=True)
    for k, e in errs.items():
        if k != "dc0":  # dc0 = the sum of dp0: checked against the kernel's own dp0
            assert e <= tol(dtype), (k, e)
    check_dc0(g["dc0"].cpu().numpy(), g["dp0"].cpu().numpy())



def test_gated_backward_with_a_pair_out_of_range(dev):
    # one (batch, head) pair has a chunk of z_alpha = -14 (alpha ~ 8e-7),
    # outside the chunked form's range: that pair takes the token path on the
    # fp32 copies of its gated values, the others the chunked path on the raw
    # inputs, in the same call
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gbwd_mix", "diagonal", "bf16", 2, 300, 2, 128, 128, 128.0, "uniform", 1790, omega_loc=-1.0)
    x = wl.gated_inputs(w)
    x["z_alpha"][1, 96:128, 0] = wl.round_bf16(np.full((32, 128), -14.0, np.float32))
    ct = wl.backward_cotangents(w, with_state=True)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev) for n in GATED}
    g = kdn.backward_gated(**t, c0=_f32(x["c0"], dev), mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev),
                           dS_T=_f32(ct["dS_T"], dev), dp_T=_f32(ct["dp_T"], dev))
    torch.cuda.synchronize()
    ref = oracle.backward_gated(**{n: x[n] for n in GATED}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                                dp_T=ct["dp_T"])
    errs = {k: rel_err(g[k].cpu().numpy(), ref[k]) for k in GRADS}
    print("gated bwd mixed range: " + " ".join(f"{k}={e:.1e}" for k, e in errs.items()), flush=True)
    for k, e in errs.items():
        if k != "dc0":
            assert e <= tol("bf16"), (k, e)
    check_dc0(g["dc0"].cpu().numpy(), g["dp0"].cpu().numpy())


def test_gated_backward_full_size_sampled_heads(dev):
    """kdn_backward_gated at B=8, T=4096, H=16, d=128 (diagonal, bf16, the
    chunked path with the gates and the q/k normalisation inside its
    kernels); the oracle runs on sampled (batch, head) pairs."""
    import torch
    import kalman_delta_network_amd as kdn
    from kdn_testutil import sample_pairs
    w = wl.WORKLOADS["diag_bf16_b8_t4096_h16_d128"]
    x = wl.gated_inputs(w)
    ct = wl.backward_cotangents(w, with_state=False)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev) for n in GATED}
    g = kdn.backward_gated(**t, c0=_f32(x["c0"], dev), mu=w.mu,
                           dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev), variant=w.variant)
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in g.items()}
    pairs = sample_pairs(w.B, w.H, 2, seed=w.seed + 1)
    worst = {k: 0.0 for k in GRADS if k != "dc0"}
    for b, h in pairs:
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in GATED}
        ref = oracle.backward_gated(**sub, c0=x["c0"][h:h + 1], mu=w.mu,
                                    dO=np.ascontiguousarray(ct["dO"][b:b + 1, :, h:h + 1]), variant=w.variant)
        for k in worst:
            gk = got[k][b:b + 1, :, h:h + 1] if k not in ("dS0", "dp0") else got[k][b:b + 1, h:h + 1]
            worst[k] = max(worst[k], rel_err(gk, ref[k]))
    print(f"gated full size pairs={pairs}: " + " ".join(f"{k}={v:.1e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (k, e)
    for k in GRADS:
        assert np.all(np.isfinite(got[k])), k
    check_dc0(got["dc0"], got["dp0"])


def test_gated_backward_misaligned_q_k(dev):
    """q and k two bytes off 16-byte alignment: the chunked path does not
    apply (it loads 16-byte pieces), so every pair takes the token path on
    the fp32 copies (read element by element), and the normalisation's
    Jacobian takes its element-wise pass instead of the 16-byte one."""
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gbwd_mis", "diagonal", "bf16", 2, 100, 2, 128, 128, 128.0, "uniform", 1811, omega_loc=-1.0)
    x = wl.gated_inputs(w)
    ct = wl.backward_cotangents(w, with_state=True)

    def misaligned(a):
        buf = torch.empty(a.size + 1, dtype=torch.bfloat16, device=dev)
        view = buf[1:].view(a.shape)
        view.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16))
        assert view.data_ptr() % 16 != 0
        return view

    t = {n: (misaligned(x[n]) if n in ("q", "k") else
             torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev)) for n in GATED}
    g = kdn.backward_gated(**t, c0=_f32(x["c0"], dev), mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev),
                           dS_T=_f32(ct["dS_T"], dev), dp_T=_f32(ct["dp_T"], dev))
    torch.cuda.synchronize()
    ref = oracle.backward_gated(**{n: x[n] for n in GATED}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                                dp_T=ct["dp_T"])
    errs = {k: rel_err(g[k].cpu().numpy(), ref[k]) for k in GRADS}
    print("gated bwd misaligned q, k: " + " ".join(f"{k}={e:.1e}" for k, e in errs.items()), flush=True)
    for k, e in errs.items():
        if k != "dc0":
            assert e <= tol("bf16"), (k, e)
    check_dc0(g["dc0"].cpu().numpy(), g["dp0"].cpu().numpy())
