"""GPU parity of the two workgroup widths of the chunked forward (64 or 32
value columns per workgroup, forced through KDN_ALGO_CHUNKED_WIDE and
KDN_ALGO_CHUNKED_NARROW) against the fp64 oracle, and of the two widths
against each other.  Every value column is computed by the same instructions
in both widths, so their outputs agree bit for bit.  Tolerance 2e-2 max
relative error (bf16 inputs, fp32 state) against the oracle."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_forward, TOKEN_INPUTS, oracle_forward, oracle_forward_heads, rel_err, sample_pairs, to_dev, tol

pytestmark = pytest.mark.gpu

WIDTHS = ["chunked_wide", "chunked_narrow"]


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _f32(a, dev):
    import torch
    return None if a is None else torch.from_numpy(np.asarray(a, np.float32)).to(dev)


def run(dev, w, x, algo, S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    o, S, p = kdn.forward(**t, mu=w.mu, variant=w.variant, S0=_f32(S0, dev), p0=_f32(p0, dev), algo=algo)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


def check(name, got, ref):
    return check_forward(name, got, ref, "bf16")


@pytest.mark.parametrize("algo", WIDTHS)
@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_width_forward(dev, algo, variant, dk, dv, T):
    w = wl.Workload("width", variant, "bf16", 2, T, 3, dk, dv, float(dk), "uniform", 1300 + T + dk + dv,
                    omega_loc=-1.0 if T % 2 else 0.0)
    x = wl.forward_inputs(w)
    check(f"{algo}/{variant}/dk{dk}/dv{dv}/T{T}", run(dev, w, x, algo), oracle_forward(w, x))


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_widths_agree_bit_for_bit(dev, variant):
    w = wl.Workload("width_eq", variant, "bf16", 3, 333, 2, 128, 128, 128.0, "uniform", 1401, omega_loc=-0.5)
    x = wl.forward_inputs(w)
    wide = run(dev, w, x, "chunked_wide")
    narrow = run(dev, w, x, "chunked_narrow")
    for key, a, b in zip(("o", "S", "p"), wide, narrow):
        assert np.array_equal(a, b), (variant, key, float(np.max(np.abs(a - b))))


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_narrow_with_initial_state(dev, variant):
    w = wl.Workload("width_init", variant, "bf16", 2, 150, 2, 128, 128, 128.0, "uniform", 1402, omega_loc=0.0)
    x = wl.forward_inputs(w)
    st = wl.decode_state(w)
    check(f"narrow/{variant}/init", run(dev, w, x, "chunked_narrow", S0=st["S0"], p0=st["p0"]),
          oracle_forward(w, x, S0=st["S0"], p0=st["p0"]))


@pytest.mark.parametrize("algo", WIDTHS)
def test_width_packed_batch(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    lengths = [1, 33, 0, 90, 64, 129]
    w = wl.Workload("width_var", "diagonal", "bf16", len(lengths), 0, 3, 128, 128, 128.0, "uniform", 1403,
                    omega_loc=-1.0)
    x = wl.varlen_inputs(w, lengths)
    t = to_dev(x, "bf16", dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    o, S, p = kdn.forward_varlen(**t, cu_seqlens=cu, mu=w.mu, algo=algo,
                                 order=torch.from_numpy(kdn.longest_first(x["cu_seqlens"])).to(dev))
    torch.cuda.synchronize()
    ref = oracle.forward_varlen(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu,
                                cu_seqlens=x["cu_seqlens"], variant="diagonal")
    check(f"{algo}/varlen", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()), ref)


def test_narrow_rejects_grouped_noise(dev):
    import kalman_delta_network_amd as kdn
    w = wl.Workload("width_grp", "grouped", "bf16", 1, 64, 1, 128, 128, 128.0, "uniform", 1404, rgroups=2)
    x = wl.forward_inputs(w)
    with pytest.raises(kdn.KDNError) as e:
        kdn.forward(**to_dev(x, "bf16", dev), mu=w.mu, variant="grouped", algo="chunked_narrow")
    assert e.value.status == kdn.KDN_ERR_UNSUPPORTED


@pytest.mark.parametrize("algo", WIDTHS)
def test_width_full_size_long_context(dev, algo):
    # one sequence of 65536 tokens, 16 heads: the shape the narrow width is for
    w = wl.WORKLOADS["diag_bf16_b1_t65536_h16_d128"]
    x = wl.forward_inputs(w)
    o, S, p = run(dev, w, x, algo)
    pairs = sample_pairs(w.B, w.H, 2, seed=w.seed)
    worst = {"o": 0.0, "S": 0.0, "p": 0.0}
    for (b, h), rr in oracle_forward_heads(w, x, pairs).items():
        got = (o[b:b + 1, :, h:h + 1], S[b:b + 1, h:h + 1], p[b:b + 1, h:h + 1])
        for key, g in zip(("o", "S", "p"), got):
            worst[key] = max(worst[key], rel_err(g, rr[key]))
    print(f"{algo}/long pairs={pairs}: " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (k, e)
