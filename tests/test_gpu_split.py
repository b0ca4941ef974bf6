"""GPU parity of the split forward (kdn_forward_split): each sequence cut into
segments that run concurrently, against the fp64 oracle on every (batch,
head) pair.  Tolerance as the other bf16 forwards (2e-2, per tensor; p also
elementwise)."""
import numpy as np
import pytest

from kalman_delta_network_amd import workloads as wl
from kdn_testutil import TOKEN_INPUTS, check_forward, oracle_forward, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _f32(x, dev):
    import torch
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)


def run_split(dev, w, x, segments, S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, "bf16", dev)
    o, S, p = kdn.forward_split(**t, mu=w.mu, S0=_f32(S0, dev), p0=_f32(p0, dev), segments=segments)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T,segments", [(1000, 3), (777, 4), (4096, 2), (96, 2)])
def test_split_matches_oracle(dev, dk, dv, T, segments):
    # segments of a multiple of 32 tokens, the last one ragged
    w = wl.Workload("split", "diagonal", "bf16", 2, T, 2, dk, dv, float(dk), "uniform", 61)
    x = wl.forward_inputs(w)
    got = run_split(dev, w, x, segments)
    check_forward(f"split/T{T}/s{segments}/{dk}x{dv}", got, oracle_forward(w, x), "bf16")


def test_split_with_initial_state(dev):
    # S0 enters the first segment; p0 reaches every segment through the
    # earlier segments' uncertainty maps
    w = wl.Workload("split_s0", "diagonal", "bf16", 2, 900, 3, 128, 128, 128.0, "uniform", 62, omega_loc=-1.0)
    x = wl.forward_inputs(w)
    st = wl.decode_state(w)
    got = run_split(dev, w, x, 3, S0=st["S0"], p0=st["p0"])
    ref = oracle_forward(w, x, S0=st["S0"].astype(np.float64), p0=st["p0"].astype(np.float64))
    check_forward("split/S0", got, ref, "bf16")


@pytest.mark.parametrize("alpha_const,chunk", [(1e-6, 12), (1e-3, 20), (1e-6, 0)])
def test_split_tiny_decay(dev, alpha_const, chunk):
    # a full chunk of tiny decay inside a later segment (or the first one):
    # its workgroups, identity columns included, finish the segment with the
    # token recurrence
    w = wl.Workload("split_tiny", "diagonal", "bf16", 1, 1024, 2, 128, 128, 128.0, "uniform", 63)
    x = wl.forward_inputs(w)
    lo = 32 * chunk
    x["alpha"][:, lo:lo + 32] = float(wl.round_bf16(np.array([alpha_const], np.float32))[0])
    got = run_split(dev, w, x, 3)
    check_forward(f"split/tiny{alpha_const}/chunk{chunk}", got, oracle_forward(w, x), "bf16")


def test_split_one_segment_is_the_forward(dev):
    # segments = 1 (or a sequence too short to cut) is the plain forward
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("split1", "diagonal", "bf16", 2, 300, 2, 128, 128, 128.0, "uniform", 64)
    x = wl.forward_inputs(w)
    t = to_dev(x, "bf16", dev)
    a = kdn.forward_split(**t, mu=w.mu, segments=1)
    b = kdn.forward(**t, mu=w.mu, algo="auto")
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_split_long_context_full_size(dev):
    # B=1, T=65536, H=16, d=128 with the device's own segment choice, every
    # head against the oracle
    w = wl.WORKLOADS["diag_bf16_b1_t65536_h16_d128"]
    x = wl.forward_inputs(w)
    got = run_split(dev, w, x, 0)
    check_forward("split/long context full size", got, oracle_forward(w, x), "bf16")
