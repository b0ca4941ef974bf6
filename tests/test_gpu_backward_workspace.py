"""The chunked backward on its own workspace (kdn_backward_workspace_size_for,
under 1 GB at B=8, T=4096, H=16, d=128): the adjoint runs over slabs of tokens
from the last, carrying the state's and the uncertainty's cotangents from one
slab to the next, and pairs on the token path run in rounds of as many as the
workspace holds.  Each case runs once on the smallest workspace and once on
the all-pairs one (a single slab, one round); the results must agree bit for
bit, and sampled pairs must match the fp64 oracle's adjoint within the bf16
tolerance (2e-2, max relative error per gradient)."""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl
from kdn_testutil import TOKEN_INPUTS, r256, rel_err, to_dev, token_pair_bytes, tol

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0")
B, T, H, D = 8, 1100, 16, 128  # three 512-token slabs (512, 512, 76) on the smallest workspace


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def _case(seed, out_of_range=(), shape=(B, T, H, D, D)):
    b_, t_, h_, dk, dv = shape
    w = wl.Workload("bwd_ws", "diagonal", "bf16", b_, t_, h_, dk, dv, float(dk), "uniform", seed, omega_loc=-1.0)
    x = wl.forward_inputs(w)
    for b, h, c in out_of_range:  # a chunk of alpha = 1e-6: the pair leaves the chunked form's range
        x["alpha"][b, 32 * c:32 * c + 32, h] = wl.round_bf16(np.full((32, dk), 1e-6, np.float32))
    ct = wl.backward_cotangents(w, with_state=True)
    rng = np.random.default_rng(seed + 1)
    st = {"S0": wl.round_bf16(rng.standard_normal((b_, h_, dk, dv)).astype(np.float32) * 0.2),
          "p0": rng.uniform(0.5, 2.0, (b_, h_, dk)).astype(np.float32)}
    return w, x, ct, st


def _run(dev, w, x, ct, st, ws_bytes, misalign=False):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, "bf16", dev)
    if misalign:  # q and k 2 bytes off 16-byte alignment: the token path takes every pair
        for n in ("q", "k"):
            buf = torch.empty(t[n].numel() + 1, dtype=torch.bfloat16, device=dev)
            buf[1:].copy_(t[n].reshape(-1))
            t[n] = buf[1:].view(t[n].shape)
            assert t[n].data_ptr() % 16 != 0
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    g = kdn.backward(**t, mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev), dS_T=f32(ct["dS_T"]),
                     dp_T=f32(ct["dp_T"]), S0=f32(st["S0"]), p0=f32(st["p0"]), workspace=ws)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in g.items()}


def _sizes(w=None):
    import torch
    import kalman_delta_network_amd as kdn
    b_, t_, h_, dk, dv = (B, T, H, D, D) if w is None else (w.B, w.T, w.H, w.dk, w.dv)
    small = kdn.backward_workspace_size(b_, t_, h_, dk, dv, "diagonal", torch.bfloat16)
    full = kdn.backward_workspace_size(b_, t_, h_, dk, dv)
    assert small < full
    return small, full


def _check_pairs(name, got, w, x, ct, st, pairs):
    """Sampled pairs against oracle.backward (bf16 tolerance), every gradient finite."""
    worst = {k: 0.0 for k in GRADS}
    for b, h in pairs:
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in TOKEN_INPUTS}
        ref = oracle.backward(**sub, c0=x["c0"][h:h + 1], mu=w.mu,
                              dO=np.ascontiguousarray(ct["dO"][b:b + 1, :, h:h + 1]),
                              dS_T=np.ascontiguousarray(ct["dS_T"][b:b + 1, h:h + 1]),
                              dp_T=np.ascontiguousarray(ct["dp_T"][b:b + 1, h:h + 1]),
                              S0=np.ascontiguousarray(st["S0"][b:b + 1, h:h + 1]),
                              p0=np.ascontiguousarray(st["p0"][b:b + 1, h:h + 1]), variant="diagonal")
        for k in GRADS:
            gk = got[k][b:b + 1, :, h:h + 1] if k not in ("dS0", "dp0") else got[k][b:b + 1, h:h + 1]
            worst[k] = max(worst[k], rel_err(gk, ref[k]))
    print(f"{name} pairs={pairs}: " + " ".join(f"{k}={v:.1e}" for k, v in worst.items()), flush=True)
    for k, e in worst.items():
        assert e <= tol("bf16"), (name, k, e)
    for k in GRADS:
        assert np.all(np.isfinite(got[k])), (name, k)


def _differing_pairs(a, b):
    """{gradient: sorted (b, h) pairs where the two runs differ}"""
    out = {}
    for n in a:
        d = a[n] != b[n]
        if d.ndim >= 3 and n not in ("dS0", "dp0", "dc0"):
            d = d.reshape(d.shape[0], d.shape[1], d.shape[2], -1).any(axis=(1, 3))
        elif n in ("dS0", "dp0"):
            d = d.reshape(d.shape[0], d.shape[1], -1).any(axis=2)
        else:
            d = d.reshape(1, -1)
        idx = np.argwhere(d)
        if idx.size:
            out[n] = [tuple(int(v) for v in r) for r in idx[:12]]
    return out


def _equal(a, b, name):
    diff = _differing_pairs(a, b)
    print(f"{name}: pairs that differ: {diff}", flush=True)
    for n in a:
        assert np.array_equal(a[n], b[n]), (name, n, float(np.max(np.abs(a[n] - b[n]))))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_backward_slabs_equal_one_slab(dev, dk, dv):
    # three slabs with dS and dp carried between them, against one slab
    w, x, ct, st = _case(5101 + dk + dv, shape=(B, T, H, dk, dv))
    small, full = _sizes(w)
    a = _run(dev, w, x, ct, st, small)
    b = _run(dev, w, x, ct, st, full)
    _equal(a, b, f"slabs/dk{dk}/dv{dv}")
    _check_pairs(f"slabs/dk{dk}/dv{dv}", a, w, x, ct, st, [(0, 0), (3, 9), (7, 15)])


def test_backward_long_sequence_slabs(dev):
    # B*H = 16 pairs: 4096-token slabs (64k token-heads), T = 10000 gives
    # three (4096, 4096, 1808), each with 64 uncertainty segments
    w, x, ct, st = _case(5105, shape=(1, 10000, 16, D, D))
    small, full = _sizes(w)
    a = _run(dev, w, x, ct, st, small)
    b = _run(dev, w, x, ct, st, full)
    _equal(a, b, "long")
    _check_pairs("long", a, w, x, ct, st, [(0, 7)])


def test_backward_token_path_rounds_for_pairs_out_of_range(dev):
    # pairs 5 and 100 (of 128) leave the chunked range; on the smallest
    # workspace the token path takes them in rounds of fewer than 128 pairs
    w, x, ct, st = _case(5102, out_of_range=[(0, 5, 3), (6, 4, 30)])
    small, full = _sizes()
    per_round = (small - r256(B * H * 4)) // token_pair_bytes(T, D, D)
    assert 1 <= per_round < B * H, per_round
    a = _run(dev, w, x, ct, st, small)
    b = _run(dev, w, x, ct, st, full)
    print("rounds: small vs small", _differing_pairs(a, _run(dev, w, x, ct, st, small)), flush=True)
    print("rounds: full vs full", _differing_pairs(b, _run(dev, w, x, ct, st, full)), flush=True)
    for tag, g in (("small", a), ("full", b)):
        try:
            _check_pairs(f"rounds/{tag}", g, w, x, ct, st, [(0, 5), (6, 4), (2, 2)])
        except AssertionError as e:
            print(f"rounds/{tag}: {e}", flush=True)
    _equal(a, b, "rounds")
    _check_pairs("rounds", a, w, x, ct, st, [(0, 5), (6, 4), (2, 2)])


def test_backward_misaligned_inputs_on_the_chunked_workspace(dev):
    # q and k off alignment send every pair to the token path, in rounds on
    # the chunked path's workspace
    w, x, ct, st = _case(5103)
    small, full = _sizes()
    a = _run(dev, w, x, ct, st, small, misalign=True)
    b = _run(dev, w, x, ct, st, full, misalign=True)
    _equal(a, b, "misaligned")
    _check_pairs("misaligned", a, w, x, ct, st, [(1, 1), (5, 12)])


def test_gated_backward_smallest_workspace_equals_all_pairs(dev):
    # kdn_backward_gated on kdn_backward_gated_workspace_size_for (the fp32
    # copies at its end, the chunked adjoint in slabs before them) and on the
    # all-pairs size, with two pairs on the token path (a chunk of z_alpha =
    # -14, alpha ~ 8e-7); the gated parity tests cover the smallest size
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("gbwd_ws", "diagonal", "bf16", B, T, H, D, D, float(D), "uniform", 5104, omega_loc=-1.0)
    x = wl.gated_inputs(w)
    for b, h, c in ((1, 3, 2), (7, 11, 33)):
        x["z_alpha"][b, 32 * c:32 * c + 32, h] = wl.round_bf16(np.full((32, D), -14.0, np.float32))
    ct = wl.backward_cotangents(w, with_state=True)
    t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16).to(dev)
         for n in ("q", "k", "v", "z_alpha", "z_omega", "z_r")}
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    small = kdn.backward_gated_workspace_size(B, T, H, D, D, "diagonal", torch.bfloat16)
    full = kdn.backward_gated_workspace_size(B, T, H, D, D, "diagonal")
    assert small < full
    out = []
    for nb in (small, full):
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        g = kdn.backward_gated(**t, c0=f32(x["c0"]), mu=w.mu, dO=torch.from_numpy(ct["dO"]).to(torch.bfloat16).to(dev),
                               dS_T=f32(ct["dS_T"]), dp_T=f32(ct["dp_T"]), workspace=ws)
        torch.cuda.synchronize()
        out.append({n: v.cpu().numpy() for n, v in g.items()})
        del ws
    _equal(out[0], out[1], "gated")
    for n, v in out[0].items():
        assert np.all(np.isfinite(v)), n
