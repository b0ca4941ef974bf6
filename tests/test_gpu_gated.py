"""GPU parity of the gated forward (kdn_forward_gated and its decode and
packed-batch forms: the step before the recurrence done inside the kernels,
q and k L2-normalised per token-head and the gates alpha = sigmoid(z),
omega = softplus(z), r = 0.01 + softplus(z), for the diagonal, isotropic and
per-channel-decay isotropic variants) against oracle.forward_gated /
oracle.prologue on the same raw q, k and pre-activations, through the C ABI.  Tolerance: max relative error 1e-4
(fp32 inputs) or 2e-2 (bf16 inputs, fp32 state), per output tensor."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_forward, rel_err, sample_pairs, tol

pytestmark = pytest.mark.gpu

GATED = ("q", "k", "v", "z_alpha", "z_omega", "z_r")


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def to_dev(x, dtype, dev):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(tdt).to(dev) for n in GATED}
    out["c0"] = torch.from_numpy(np.ascontiguousarray(x["c0"], np.float32)).to(dev)
    return out


def run(dev, w, x, algo, S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    f32 = (lambda a: None if a is None else torch.from_numpy(np.asarray(a, np.float32)).to(dev))
    o, S, p = kdn.forward_gated(**to_dev(x, w.dtype, dev), mu=w.mu, variant=w.variant, S0=f32(S0), p0=f32(p0),
                                algo=algo)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


def oracle_gated(w, x, S0=None, p0=None):
    return oracle.forward_gated(**{n: x[n] for n in GATED}, c0=x["c0"], mu=w.mu, S0=S0, p0=p0, variant=w.variant)


def check(name, got, ref, dtype):
    return check_forward(name, got, ref, dtype)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("algo", ["recurrent", "chunked_wide", "chunked_narrow"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_gated_forward(dev, variant, algo, dtype, dk, dv, T):
    if dtype == "f32" and algo != "recurrent":
        pytest.skip("the chunked kernel takes bf16 inputs")
    # omega_loc 0: softplus near its bend, z_alpha around 2 (decay ~0.88)
    w = wl.Workload("gated", variant, dtype, 2, T, 3, dk, dv, float(dk), "uniform", 1500 + T + dk + dv,
                    omega_loc=0.0 if T % 2 else -4.0)
    x = wl.gated_inputs(w)
    assert x["z_r"].shape == (2, T, 3)
    assert x["z_alpha"].shape == ((2, T, 3) if variant == "isotropic" else (2, T, 3, dk))
    assert x["z_omega"].shape == ((2, T, 3, dk) if variant == "diagonal" else (2, T, 3))
    check(f"gated/{variant}/{algo}/{dtype}/dk{dk}/dv{dv}/T{T}", run(dev, w, x, algo), oracle_gated(w, x), dtype)


def test_gated_extreme_pre_activations(dev):
    # pre-activations far in the tails: softplus at 0 and at z, r at its floor
    # 0.01, the decay anywhere from saturated at 1 to about 1e-30 (the chunked
    # kernel hands such chunks to the token recurrence)
    w = wl.Workload("gated_ext", "diagonal", "bf16", 2, 97, 2, 128, 128, 128.0, "uniform", 1601)
    x = wl.gated_inputs(w)
    rng = np.random.default_rng(5)
    for n, s in (("z_alpha", 30.0), ("z_omega", 30.0), ("z_r", 30.0)):
        x[n] = wl.round_bf16(rng.normal(0.0, s, size=x[n].shape).astype(np.float32))
    for algo in ("recurrent", "chunked"):
        check(f"gated/extreme/{algo}", run(dev, w, x, algo), oracle_gated(w, x), "bf16")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_gated_small_process_noise_f32(dev, variant):
    # z_omega ~ N(-10, 1): softplus(z) ~ e^z, where rounding 1 + e^z alone
    # would lose the value; fp32 tolerance 1e-4 on every output
    w = wl.Workload("gated_small_omega", variant, "f32", 2, 70, 2, 128, 128, 128.0, "uniform", 1606,
                    omega_loc=-10.0)
    x = wl.gated_inputs(w)
    check(f"gated/small_omega/{variant}", run(dev, w, x, "recurrent"), oracle_gated(w, x), "f32")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_gated_with_initial_state(dev, variant, algo):
    w = wl.Workload("gated_init", variant, "bf16", 2, 150, 2, 128, 128, 128.0, "uniform", 1602, omega_loc=-1.0)
    x = wl.gated_inputs(w)
    st = wl.decode_state(w)
    check(f"gated/init/{variant}/{algo}", run(dev, w, x, algo, S0=st["S0"], p0=st["p0"]),
          oracle_gated(w, x, S0=st["S0"], p0=st["p0"]), "bf16")


def test_gated_rejects_grouped_noise(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gated_var", "diagonal", "bf16", 1, 8, 1, 128, 128, 128.0, "uniform", 1603)
    t = to_dev(wl.gated_inputs(w), "bf16", dev)
    o = torch.empty((1, 8, 1, 128), dtype=torch.bfloat16, device=dev)
    S = torch.empty((1, 1, 128, 128), dtype=torch.float32, device=dev)
    p = torch.empty((1, 1), dtype=torch.float32, device=dev)
    lib = kdn.load_library()
    st = lib.kdn_forward_gated(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["z_alpha"].data_ptr(),
                               t["z_omega"].data_ptr(), t["z_r"].data_ptr(), t["c0"].data_ptr(), 128.0,
                               kdn.KDN_DIAGONAL_GROUPED, 1, 1, 8, 1, 128, 128, None, None, o.data_ptr(), S.data_ptr(),
                               p.data_ptr(), None, 0)
    assert st == kdn.KDN_ERR_UNSUPPORTED


def test_gated_full_size_sampled_heads(dev):
    # the main forward's shape (B=8, T=4096, H=16, d=128, bf16) through the gates,
    # in the launch configuration the benchmark times; oracle on sampled heads
    w = wl.WORKLOADS["diag_bf16_b8_t4096_h16_d128"]
    x = wl.gated_inputs(w)
    o, S, p = run(dev, w, x, "auto")
    worst = {"o": 0.0, "S": 0.0, "p": 0.0}
    pairs = sample_pairs(w.B, w.H, 4, seed=w.seed)
    for b, h in pairs:
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in GATED}
        rr = oracle.forward_gated(**sub, c0=x["c0"][h:h + 1], mu=w.mu)
        got = (o[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1], p[b:b + 1, h:h + 1])
        for key, g in zip(("o", "S", "p"), got):
            worst[key] = max(worst[key], rel_err(g, rr[key]))
    print(f"gated full size pairs={pairs}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (k, e)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_gated_decode_steps(dev, variant):
    # four consecutive decode steps from pre-activations; token s of each
    # sequence is position s of a gated input draw
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gated_dec", variant, "bf16", 8, 4, 4, 128, 128, 128.0, "uniform", 1604, omega_loc=-1.0)
    x = wl.gated_inputs(w)
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    Sr, pr = st["S0"].astype(np.float64), st["p0"].astype(np.float64)
    for s in range(w.T):
        tok = {n: np.ascontiguousarray(x[n][:, s]) for n in GATED}
        t = {n: torch.from_numpy(tok[n]).to(torch.bfloat16).to(dev) for n in GATED}
        o = kdn.step_gated(**t, mu=w.mu, S=S, p=p, variant=variant)
        qh, kh, a, om, r = oracle.prologue(tok["q"], tok["k"], tok["z_alpha"], tok["z_omega"], tok["z_r"])
        fn = {"diagonal": oracle.step_diag, "isotropic": oracle.step_iso, "isochannel": oracle.step_isoc}[variant]
        ref = fn(qh, kh, tok["v"], a, om, r, mu=w.mu, S=Sr, p=pr)
        Sr, pr = ref["S"], ref["p"]
        torch.cuda.synchronize()
        check(f"gated/decode/{variant}/step{s}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()),
              {"o": ref["o"], "S": Sr, "p": pr}, "bf16")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_gated_packed_batch(dev, variant, algo):
    import torch
    import kalman_delta_network_amd as kdn
    lengths = [1, 33, 0, 90, 64, 129]
    total = sum(lengths)
    w = wl.Workload("gated_var", variant, "bf16", 1, total, 3, 128, 128, 128.0, "uniform", 1605, omega_loc=-1.0)
    x = {n: (v[0] if n != "c0" else v) for n, v in wl.gated_inputs(w).items()}  # [total, H, *]
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev) for n in GATED}
    o, S, p = kdn.forward_varlen_gated(**t, c0=torch.from_numpy(x["c0"]).to(dev),
                                       cu_seqlens=torch.from_numpy(cu).to(dev), mu=w.mu, variant=variant, algo=algo,
                                       order=torch.from_numpy(kdn.longest_first(cu)).to(dev))
    torch.cuda.synchronize()
    qh, kh, a, om, r = oracle.prologue(x["q"], x["k"], x["z_alpha"], x["z_omega"], x["z_r"])
    ref = oracle.forward_varlen(qh, kh, x["v"], a, om, r, c0=x["c0"], mu=w.mu, cu_seqlens=cu, variant=variant)
    check(f"gated/varlen/{variant}/{algo}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref, "bf16")
