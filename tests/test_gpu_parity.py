"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
identical seeded inputs.  Tolerance: max relative error 1e-4 (fp32 inputs)
or 2e-2 (bf16 inputs, fp32 state), per output tensor."""
import numpy as np
import pytest

from kalman_delta_network_amd import workloads as wl
from kdn_testutil import (check_forward, TOKEN_INPUTS, oracle_forward, oracle_forward_heads, rel_err, sample_pairs,
                          to_dev, tol)

pytestmark = pytest.mark.gpu

ALGOS = ["recurrent", "chunked"]


@pytest.fixture(scope="module")
def dev():
    import torch
    import kalman_delta_network_amd as kdn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kdn.load_library()
    return torch.device("cuda:0")


def run_forward(dev, w, x, algo, S0=None, p0=None):
    import torch
    import kalman_delta_network_amd as kdn
    t = to_dev(x, w.dtype, dev)
    S0d = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).to(dev)
    p0d = None if p0 is None else torch.from_numpy(np.asarray(p0, np.float32)).to(dev)
    try:
        o, S, p = kdn.forward(**t, mu=w.mu, variant=w.variant, S0=S0d, p0=p0d, algo=algo)
    except kdn.KDNError as e:
        if e.status == kdn.KDN_ERR_UNSUPPORTED and algo == "chunked":
            pytest.skip("chunked algorithm does not cover this shape")
        raise
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()


def check(name, got, ref, dtype):
    return check_forward(name, got, ref, dtype)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_forward_small(dev, algo, variant, dtype, dk, dv, T):
    w = wl.Workload("small", variant, dtype, 2, T, 3, dk, dv, float(dk), "uniform",
                    100 + T + dk + dv, omega_loc=-4.0 if T % 2 else 0.0)
    x = wl.forward_inputs(w)
    got = run_forward(dev, w, x, algo)
    check(f"{algo}/{variant}/{dtype}/dk{dk}/dv{dv}/T{T}", got, oracle_forward(w, x), dtype)


# Shapes that exercise the chunked kernel's work mapping and range: more than
# eight (batch, head) items (a ragged last group of XCD-dealt items), a
# single head, batch counts that are not multiples of 8, one-token tails, and
# strong decay (alpha ~ sigmoid(N(0, 0.5)) or sigmoid(N(-1, 0.5)), so the
# in-chunk cumulative decay reaches 1e-10 .. 1e-18).
SHAPES = [
    # B, T, H, dk, dv, alpha_loc, omega_loc
    (9, 97, 2, 128, 128, 0.0, -1.0),
    (1, 130, 1, 64, 64, 2.0, -4.0),
    (16, 40, 1, 128, 64, -1.0, -2.0),
]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}_t{}_h{}_dk{}_dv{}_a{}".format(*s[:6]))
def test_forward_shapes(dev, algo, variant, shape):
    B, T, H, dk, dv, aloc, oloc = shape
    w = wl.Workload("shape", variant, "bf16", B, T, H, dk, dv, float(dk), "uniform",
                    700 + B + T + H + dv, alpha_loc=aloc, omega_loc=oloc)
    x = wl.forward_inputs(w)
    got = run_forward(dev, w, x, algo)
    check(f"{algo}/{variant}/b{B}/t{T}/h{H}/dk{dk}/dv{dv}/a{aloc}", got, oracle_forward(w, x), "bf16")


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_forward_with_initial_state(dev, algo, variant):
    w = wl.Workload("init", variant, "bf16", 3, 150, 2, 128, 128, 128.0, "uniform", 77, omega_loc=0.0)
    x = wl.forward_inputs(w)
    st = wl.decode_state(w.with_(B=3))
    got = run_forward(dev, w, x, algo, S0=st["S0"], p0=st["p0"])
    check(f"{algo}/{variant}/init", got, oracle_forward(w, x, S0=st["S0"], p0=st["p0"]), "bf16")


@pytest.mark.parametrize("algo", ALGOS)
def test_isotropic_write_heavy_case(dev, algo):
    # extra isotropic case with larger process noise, so that writes are not tiny
    w = wl.Workload("iso_heavy", "isotropic", "bf16", 2, 300, 4, 128, 128, 128.0, "uniform", 91,
                    omega_loc=0.0)
    x = wl.forward_inputs(w)
    check(f"{algo}/iso_heavy", run_forward(dev, w, x, algo), oracle_forward(w, x), "bf16")


@pytest.mark.parametrize("algo", ALGOS)
def test_split_continuation(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("split", "diagonal", "bf16", 2, 190, 2, 128, 128, 128.0, "uniform", 55)
    x = wl.forward_inputs(w)
    t = to_dev(x, "bf16", dev)
    try:
        o_full, S_full, p_full = kdn.forward(**t, mu=w.mu, algo=algo)
    except kdn.KDNError as e:
        if e.status == kdn.KDN_ERR_UNSUPPORTED:
            pytest.skip("chunked algorithm does not cover this shape")
        raise
    a = {n: t[n][:, :77].contiguous() for n in TOKEN_INPUTS}
    b = {n: t[n][:, 77:].contiguous() for n in TOKEN_INPUTS}
    o1, S1, p1 = kdn.forward(**a, c0=t["c0"], mu=w.mu, algo=algo)
    o2, S2, p2 = kdn.forward(**b, c0=None, mu=w.mu, S0=S1, p0=p1, algo=algo)
    torch.cuda.synchronize()
    ref = oracle_forward(w, x)
    got = (torch.cat([o1, o2], 1).float().cpu().numpy(), S2.cpu().numpy(), p2.cpu().numpy())
    check(f"{algo}/split", got, ref, "bf16")
    # in-place continuation: S_T is the S0 buffer
    o3, S3, p3 = kdn.forward(**b, c0=None, mu=w.mu, S0=S1, p0=p1, algo=algo, out=(
        torch.empty_like(o2), S1, torch.empty_like(p1)))
    torch.cuda.synchronize()
    assert torch.equal(S3, S2) and torch.equal(o3, o2) and torch.equal(p3, p2)


@pytest.mark.parametrize("algo", ALGOS)
def test_deterministic(dev, algo):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("det", "diagonal", "bf16", 2, 257, 4, 128, 128, 128.0, "uniform", 66)
    t = to_dev(wl.forward_inputs(w), "bf16", dev)
    try:
        r1 = kdn.forward(**t, mu=w.mu, algo=algo)
    except kdn.KDNError as e:
        if e.status == kdn.KDN_ERR_UNSUPPORTED:
            pytest.skip("chunked algorithm does not cover this shape")
        raise
    r2 = kdn.forward(**t, mu=w.mu, algo=algo)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_empty_inputs(dev):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("empty", "diagonal", "bf16", 2, 0, 3, 128, 128, 128.0, "uniform", 1)
    x = wl.forward_inputs(w)
    t = to_dev(x, "bf16", dev)
    o, S, p = kdn.forward(**t, mu=w.mu)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128)
    assert torch.count_nonzero(S).item() == 0
    np.testing.assert_array_equal(p.cpu().numpy(), np.broadcast_to(x["c0"][None, :, None], (2, 3, 128)))
    w0 = w.with_(B=0, T=5)
    t0 = to_dev(wl.forward_inputs(w0), "bf16", dev)
    o, S, p = kdn.forward(**t0, mu=w.mu)
    torch.cuda.synchronize()
    assert o.numel() == 0 and S.numel() == 0


# ---------------------------------------------------------------------------
# the workloads at their full sizes, in the launch configuration the
# benchmark times; the oracle runs on a sample of (b, h) pairs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("name", ["diag_f32_b1_t256_h2_d64", "diag_bf16_b8_t4096_h16_d128",
                                  "iso_bf16_b8_t4096_h16_d128", "diag_bf16_b1_t65536_h16_d128"])
def test_workload_full_size(dev, algo, name):
    # every (batch, head) pair of the workload against the oracle: the
    # per-tensor metric over the whole output, the same metric for each pair
    # on its own (the worst pair is printed), and p elementwise
    w = wl.WORKLOADS[name]
    x = wl.forward_inputs(w)
    o, S, p = run_forward(dev, w, x, algo)
    ref = oracle_forward(w, x)
    errs = check_forward(f"{algo}/{name} all heads", (o, S, p), ref, w.dtype)
    worst = {"o": (0.0, None), "S": (0.0, None), "p": (0.0, None)}
    for b in range(w.B):
        for h in range(w.H):
            got = {"o": o[b, :, h], "S": S[b, h], "p": p[b, h]}
            want = {"o": ref["o"][b, :, h], "S": ref["S"][b, h], "p": ref["p"][b, h]}
            for key in worst:
                e = rel_err(got[key], want[key])
                if e > worst[key][0]:
                    worst[key] = (e, (b, h))
    print(f"{algo}/{name} worst single head: " +
          " ".join(f"{k}={v[0]:.2e}@{v[1]}" for k, v in worst.items()), flush=True)
    for k, (e, where) in worst.items():
        assert e <= tol(w.dtype), (name, k, e, where)
    assert errs["p_elem"] <= tol(w.dtype) and np.all(p > 0)


@pytest.mark.parametrize("name", ["decode_diag_bf16_n256_h16_d128_s1024", "decode_iso_bf16_n256_h16_d128_s1024"])
def test_decode_full_size(dev, name):
    # 1024 plain kdn_step calls at N=256, H=16, d=128 from a carried state,
    # six sampled (sequence, head) pairs stepped by the oracle alongside
    import torch
    import kalman_delta_network_amd as kdn
    import oracle
    w = wl.WORKLOADS[name]
    ostep = oracle.step_diag if w.variant == "diagonal" else oracle.step_iso
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    pairs = sample_pairs(w.B, w.H, 6, seed=w.seed)
    Sr = {pr: st["S0"][pr[0]:pr[0] + 1, pr[1]:pr[1] + 1].astype(np.float64) for pr in pairs}
    prr = {pr: st["p0"][pr[0]:pr[0] + 1, pr[1]:pr[1] + 1].astype(np.float64) for pr in pairs}
    worst = 0.0
    for s in range(w.decode_steps):
        x = wl.decode_tokens(w, s)
        o = kdn.step(**to_dev(x, "bf16", dev), mu=w.mu, S=S, p=p, variant=w.variant)
        if s % 128 == 127 or s == w.decode_steps - 1:
            o_h = o.float().cpu().numpy()
        for pr in pairs:
            n, h = pr
            sub = {k: np.ascontiguousarray(x[k][n:n + 1, h:h + 1]) for k in TOKEN_INPUTS}
            res = ostep(**sub, mu=w.mu, S=Sr[pr], p=prr[pr])
            Sr[pr], prr[pr] = res["S"], res["p"]
            if s % 128 == 127 or s == w.decode_steps - 1:
                worst = max(worst, rel_err(o_h[n:n + 1, h:h + 1], res["o"]))
    torch.cuda.synchronize()
    S_h, p_h = S.cpu().numpy(), p.cpu().numpy()
    eS = max(rel_err(S_h[n:n + 1, h:h + 1], Sr[(n, h)]) for n, h in pairs)
    ep = max(rel_err(p_h[n:n + 1, h:h + 1], prr[(n, h)]) for n, h in pairs)
    print(f"decode full {w.variant}: o={worst:.2e} S={eS:.2e} p={ep:.2e}", flush=True)
    assert max(worst, eS, ep) <= tol("bf16")


@pytest.mark.parametrize("name", ["decode_diag_bf16_n256_h16_d128_s1024", "decode_iso_bf16_n256_h16_d128_s1024"])
def test_decode_streamed_state(dev, name):
    # N=512 sequences x 16 heads: a 537 MB state, above the size from which
    # the step streams S with nontemporal hints; 16 steps, sampled pairs
    # stepped by the oracle alongside
    import torch
    import kalman_delta_network_amd as kdn
    import oracle
    w = wl.WORKLOADS[name].with_(name=name.replace("n256", "n512"), B=512, decode_steps=16)
    ostep = oracle.step_diag if w.variant == "diagonal" else oracle.step_iso
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    pairs = sample_pairs(w.B, w.H, 6, seed=w.seed + 3)
    Sr = {pr: st["S0"][pr[0]:pr[0] + 1, pr[1]:pr[1] + 1].astype(np.float64) for pr in pairs}
    prr = {pr: st["p0"][pr[0]:pr[0] + 1, pr[1]:pr[1] + 1].astype(np.float64) for pr in pairs}
    worst = 0.0
    for s in range(w.decode_steps):
        x = wl.decode_tokens(w, s)
        o = kdn.step(**to_dev(x, "bf16", dev), mu=w.mu, S=S, p=p, variant=w.variant)
        o_h = o.float().cpu().numpy()
        for pr in pairs:
            n, h = pr
            sub = {k: np.ascontiguousarray(x[k][n:n + 1, h:h + 1]) for k in TOKEN_INPUTS}
            res = ostep(**sub, mu=w.mu, S=Sr[pr], p=prr[pr])
            Sr[pr], prr[pr] = res["S"], res["p"]
            worst = max(worst, rel_err(o_h[n:n + 1, h:h + 1], res["o"]))
    torch.cuda.synchronize()
    S_h, p_h = S.cpu().numpy(), p.cpu().numpy()
    eS = max(rel_err(S_h[n:n + 1, h:h + 1], Sr[(n, h)]) for n, h in pairs)
    ep = max(rel_err(p_h[n:n + 1, h:h + 1], prr[(n, h)]) for n, h in pairs)
    print(f"decode streamed {w.variant}: o={worst:.2e} S={eS:.2e} p={ep:.2e}", flush=True)
    assert max(worst, eS, ep) <= tol("bf16")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_decode_steps_all_heads(dev, variant):
    # eight plain kdn_step calls from a carried state (N=5, H=3, d_k=d_v=128),
    # every (sequence, head) pair against the oracle's step after each call
    import torch
    import kalman_delta_network_amd as kdn
    import oracle
    w = wl.Workload("stepall", variant, "bf16", 5, 1, 3, 128, 128, 128.0, "one", 45, omega_loc=0.0,
                    decode_steps=8)
    ostep = oracle.step_diag if variant == "diagonal" else oracle.step_iso
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    Sr, pr = st["S0"].astype(np.float64), st["p0"].astype(np.float64)
    for s in range(w.decode_steps):
        x = wl.decode_tokens(w, s)
        o = kdn.step(**to_dev(x, "bf16", dev), mu=w.mu, S=S, p=p, variant=variant)
        res = ostep(**{k: x[k] for k in TOKEN_INPUTS}, mu=w.mu, S=Sr, p=pr)
        Sr, pr = res["S"], res["p"]
        check(f"step/{variant}/{s}", (o.float().cpu().numpy(), S.cpu().numpy(), p.cpu().numpy()),
              {"o": res["o"], "S": Sr, "p": pr}, "bf16")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_steps_equal_forward(dev, variant):
    import torch
    import kalman_delta_network_amd as kdn
    w = wl.Workload("stepfwd", variant, "bf16", 3, 40, 2, 128, 128, 128.0, "uniform", 44, omega_loc=0.0)
    x = wl.forward_inputs(w)
    t = to_dev(x, "bf16", dev)
    o_f, S_f, p_f = kdn.forward(**t, mu=w.mu, variant=variant, algo="recurrent")
    S = torch.zeros_like(S_f)
    p = (t["c0"][None, :, None].expand(3, 2, 128) if variant == "diagonal" else t["c0"][None, :].expand(3, 2)).contiguous()
    outs = []
    for s in range(w.T):
        outs.append(kdn.step(**{n: t[n][:, s].contiguous() for n in TOKEN_INPUTS}, mu=w.mu, S=S, p=p,
                             variant=variant))
    torch.cuda.synchronize()
    # same kernel, same arithmetic order: bit-identical
    assert torch.equal(torch.stack(outs, 1), o_f)
    assert torch.equal(S, S_f) and torch.equal(p, p_f)
