"""GPU parity of the packed variable-length forward (kdn_forward_varlen)
against the fp64 oracle, and its agreement with the [B,T,H] forward.
Tolerances as in test_gpu_parity: 1e-4 (fp32 inputs) / 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import check_forward, TOKEN_INPUTS, rel_err, to_dev, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _state(w, N, seed):
    rng = np.random.default_rng(seed)
    S0 = (rng.standard_normal((N, w.H, w.dk, w.dv)) * 0.1).astype(np.float32)
    p0 = rng.uniform(0.1, 1.0, (N, w.H, w.dk) if w.variant == "diagonal" else (N, w.H)).astype(np.float32)
    return S0, p0


def run_varlen(dev, w, x, algo, S0=None, p0=None, order=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    S0d = None if S0 is None else torch.from_numpy(S0).to(dev)
    p0d = None if p0 is None else torch.from_numpy(p0).to(dev)
    od = None if order is None else torch.from_numpy(np.asarray(order, np.int32)).to(dev)
    try:
        o, S, p = kdn.forward_varlen(**t, cu_seqlens=cu, mu=w.mu, variant=w.variant, S0=S0d, p0=p0d, algo=algo,
                                     order=od)
    except kdn.KDNError as e:
        if e.status == kdn.KDN_ERR_UNSUPPORTED and algo == "chunked":
            pytest.skip("chunked algorithm does not cover this dtype")
        raise
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


def check(name, got, ref, dtype):
    return check_forward(name, got, ref, dtype)


# lengths around the 32-token chunk (1, 31, 32, 33, 64, 65), an empty
# sequence, and longer ones
LENGTHS = [1, 31, 32, 0, 33, 77, 200, 64, 65]


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_varlen_matches_oracle(dev, algo, variant, dtype, dk, dv):
    w = wl.Workload("varlen", variant, dtype, len(LENGTHS), 0, 3, dk, dv, float(dk), "uniform",
                    300 + dk + dv, omega_loc=-1.0)
    x = wl.varlen_inputs(w, LENGTHS)
    S0, p0 = _state(w, len(LENGTHS), 5)
    got = run_varlen(dev, w, x, algo, S0, p0)
    ref = oracle.forward_varlen(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu,
                                cu_seqlens=x["cu_seqlens"], variant=variant, S0=S0, p0=p0)
    check(f"varlen/{algo}/{variant}/{dtype}/dk{dk}/dv{dv}", got, ref, dtype)


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_varlen_equal_lengths_is_the_batched_forward(dev, algo, variant):
    # B sequences of one length, packed, give the [B,T,H] forward's outputs bit for bit
    import torch
    import kalman_delta_network_amd as kdn
    B, T = 5, 77
    w = wl.Workload("varlen_eq", variant, "bf16", B, 0, 4, 128, 128, 128.0, "uniform", 41)
    x = wl.varlen_inputs(w, [T] * B)
    got = run_varlen(dev, w, x, algo)
    t = to_dev(x, "bf16", dev)
    tb = {n: (v.reshape((B, T) + tuple(v.shape[1:])) if n in TOKEN_INPUTS else v) for n, v in t.items()}
    o, S, p = kdn.forward(**tb, mu=w.mu, variant=variant, algo=algo)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[0], o.float().cpu().numpy().reshape(got[0].shape))
    np.testing.assert_array_equal(got[1], S.cpu().numpy())
    np.testing.assert_array_equal(got[2], p.cpu().numpy())


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_varlen_scheduling_order_does_not_change_results(dev, algo, variant):
    import kalman_delta_network_amd as kdn
    w = wl.Workload("varlen_ord", variant, "bf16", len(LENGTHS), 0, 3, 128, 128, 128.0, "uniform", 43)
    x = wl.varlen_inputs(w, LENGTHS)
    S0, p0 = _state(w, len(LENGTHS), 7)
    base = run_varlen(dev, w, x, algo, S0, p0)
    for order in (kdn.longest_first(x["cu_seqlens"]), np.random.default_rng(1).permutation(len(LENGTHS))):
        got = run_varlen(dev, w, x, algo, S0, p0, order=order)
        for g, b in zip(got, base):
            np.testing.assert_array_equal(g, b)


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_varlen_all_sequences_empty(dev, algo, variant):
    w = wl.Workload("varlen_empty", variant, "bf16", 3, 0, 2, 128, 128, 128.0, "uniform", 42)
    x = wl.varlen_inputs(w, [0, 0, 0])
    S0, p0 = _state(w, 3, 6)
    o, S, p = run_varlen(dev, w, x, algo, S0, p0)
    assert o.shape == (0, 2, 128)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_array_equal(p, p0)


def test_varlen_serving_batch_sampled(dev):
    # the benchmark's packed batch (32 sequences of 256..1792 tokens, 16 heads,
    # d = 128), in the launch configuration bench.py times (longest first);
    # the oracle checks a sample of (sequence, head) pairs
    import kalman_delta_network_amd as kdn
    w = wl.VARLEN
    lengths = wl.varlen_lengths(w.seed, w.B, *wl.VARLEN_RANGE)
    x = wl.varlen_inputs(w, lengths)
    o, S, p = run_varlen(dev, w, x, "auto", order=kdn.longest_first(x["cu_seqlens"]))
    cu = x["cu_seqlens"]
    rng = np.random.default_rng(3)
    for n, h in [(0, 0), (w.B - 1, w.H - 1)] + [(int(a), int(b)) for a, b in
                                               zip(rng.integers(0, w.B, 3), rng.integers(0, w.H, 3))]:
        a, b = int(cu[n]), int(cu[n + 1])
        sub = {k: x[k][a:b, h:h + 1][None] for k in TOKEN_INPUTS}
        ref = oracle.forward_diag(**sub, c0=x["c0"][h:h + 1], mu=w.mu)
        got = (o[a:b, h:h + 1][None], S[n:n + 1, h:h + 1], p[n:n + 1, h:h + 1])
        check(f"varlen_serving/seq{n}/len{b - a}/h{h}", got, ref, "bf16")
