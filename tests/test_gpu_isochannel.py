"""GPU parity of the isotropic variant with per-channel decay
(KDN_ISOTROPIC_CHANNEL: memory decay diag(alpha), uncertainty scalar predicted
with a = mean_i alpha_i^2) against the fp64 oracle, on the recurrent and the
chunked kernels (the chunked one takes bf16 inputs only).
Tolerances 1e-4 (fp32 inputs) / 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import (check_forward, TOKEN_INPUTS, oracle_forward, oracle_forward_heads, rel_err, sample_pairs,
                          to_dev, tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def check(name, got, ref, dtype):
    return check_forward(name, got, ref, dtype)


def run(dev, w, x, algo="auto", S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    S0d = None if S0 is None else torch.from_numpy(S0).to(dev)
    p0d = None if p0 is None else torch.from_numpy(p0).to(dev)
    try:
        o, S, p = kdn.forward(**t, mu=w.mu, variant="isochannel", S0=S0d, p0=p0d, algo=algo)
    except kdn.KDNError as e:
        if e.status == kdn.KDN_ERR_UNSUPPORTED and algo == "chunked" and w.dtype == "f32":
            pytest.skip("the chunked kernel takes bf16 inputs")
        raise
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


@pytest.mark.parametrize("algo", ["auto", "recurrent", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_isochannel_forward(dev, algo, dtype, dk, dv, T):
    # omega ~ softplus(N(0, 1)): writes are not tiny; alpha ~ sigmoid(N(1, .5)) decays visibly
    w = wl.Workload("isoch", "isochannel", dtype, 2, T, 3, dk, dv, float(dk), "uniform", 900 + T + dk + dv,
                    alpha_loc=1.0, omega_loc=0.0)
    x = wl.forward_inputs(w)
    assert x["alpha"].shape == (2, T, 3, dk) and x["omega"].shape == (2, T, 3)
    check(f"isoch/{algo}/{dtype}/dk{dk}/dv{dv}/T{T}", run(dev, w, x, algo), oracle_forward(w, x), dtype)


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_isochannel_with_initial_state(dev, algo):
    w = wl.Workload("isoch_init", "isochannel", "bf16", 3, 150, 2, 128, 128, 128.0, "uniform", 78, omega_loc=0.0)
    x = wl.forward_inputs(w)
    st = wl.decode_state(w.with_(B=3))
    assert st["p0"].shape == (3, 2)
    check(f"isoch/init/{algo}", run(dev, w, x, algo, S0=st["S0"], p0=st["p0"]),
          oracle_forward(w, x, S0=st["S0"], p0=st["p0"]), "bf16")


@pytest.mark.parametrize("shape", [(9, 97, 2, 128, 128, 0.0), (16, 40, 1, 128, 64, -1.0), (1, 130, 1, 64, 64, 2.0)],
                         ids=lambda s: "b{}_t{}_h{}_dk{}_dv{}_a{}".format(*s))
def test_isochannel_chunked_shapes(dev, shape):
    # ragged item groups, one head, strong per-channel decay
    B, T, H, dk, dv, aloc = shape
    w = wl.Workload("isoch_shape", "isochannel", "bf16", B, T, H, dk, dv, float(dk), "uniform", 950 + B + T,
                    alpha_loc=aloc, omega_loc=-1.0)
    x = wl.forward_inputs(w)
    check(f"isoch/chunked/b{B}/t{T}/h{H}/dk{dk}/dv{dv}/a{aloc}", run(dev, w, x, "chunked"),
          oracle_forward(w, x), "bf16")


def test_isochannel_decode_steps(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("isoch_dec", "isochannel", "bf16", 8, 1, 4, 128, 128, 128.0, "one", 80, omega_loc=0.0)
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    Sr, pr = st["S0"].astype(np.float64), st["p0"].astype(np.float64)
    for s in range(4):
        x = wl.decode_tokens(w, s)
        assert x["alpha"].shape == (8, 4, 128) and x["omega"].shape == (8, 4)
        t = {n: torch.from_numpy(x[n]).to(torch.bfloat16).to(dev) for n in TOKEN_INPUTS}
        o = kdn.step(**t, mu=w.mu, S=S, p=p, variant="isochannel")
        ref = oracle.step_isoc(**x, mu=w.mu, S=Sr, p=pr)
        Sr, pr = ref["S"], ref["p"]
        torch.cuda.synchronize()
        check(f"isoch/decode/step{s}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()),
              {"o": ref["o"], "S": Sr, "p": pr}, "bf16")


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_isochannel_packed_batch(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    lengths = [1, 33, 0, 90, 64]
    w = wl.Workload("isoch_var", "isochannel", "bf16", len(lengths), 0, 3, 128, 128, 128.0, "uniform", 81,
                    omega_loc=0.0)
    x = wl.varlen_inputs(w, lengths)
    t = to_dev(x, "bf16", dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    o, S, p = kdn.forward_varlen(**t, cu_seqlens=cu, mu=w.mu, variant="isochannel", algo=algo,
                                 order=torch.from_numpy(kdn.longest_first(x["cu_seqlens"])).to(dev))
    torch.cuda.synchronize()
    ref = oracle.forward_varlen(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu,
                                cu_seqlens=x["cu_seqlens"], variant="isochannel")
    check(f"isoch/varlen/{algo}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref, "bf16")


def test_isochannel_full_size_sampled(dev):
    # the benchmark's workload (B=8, T=4096, H=16, d=128) in the configuration
    # bench.py times; the oracle runs on sampled heads
    w = wl.WORKLOADS["isoch_bf16_b8_t4096_h16_d128"]
    x = wl.forward_inputs(w)
    o, S, p = run(dev, w, x)
    pairs = sample_pairs(w.B, w.H, 3, seed=2)
    refs = oracle_forward_heads(w, x, pairs)
    for (b, h), ref in refs.items():
        got = (o[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1], p[b:b + 1, h:h + 1])
        check(f"isoch/full/b{b}/h{h}", got, ref, "bf16")
