"""CPU tests of the C ABI boundary: the library loads, exports every symbol
that include/kdn.h declares, and its host-side validation returns the right
status for each kind of bad argument.  No call here touches a GPU."""
import ctypes
import os
import re

import pytest

import kalman_delta_network_amd as kdn
from kdn_testutil import chunk_min_bytes, r256, token_pair_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdn.h")

MiB = 1 << 20


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kdn.LIB_PATH):
        import __graft_entry__  # noqa: F401  (build() compiles the library)
        __graft_entry__.build()
    return kdn.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(kdn.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kdn_version() == 600


def test_status_strings(lib):
    for s in range(8):
        assert lib.kdn_status_string(s)
    assert lib.kdn_status_string(99) == b"unknown status"


class Fake:
    """Distinct fake device addresses, far apart, never dereferenced."""

    def __init__(self):
        self.base = 1 << 40

    def __call__(self):
        self.base += 1 << 36
        return ctypes.c_void_p(self.base)


def fwd_args(fake, B=2, T=8, H=2, dk=64, dv=64, variant=0, dtype=1, mu=64.0, algo=0, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), omega=fake(), r=fake(), c0=fake(), mu=mu,
             variant=variant, dtype=dtype, B=B, T=T, H=H, dk=dk, dv=dv, S0=None, p0=None, o=fake(),
             S_T=fake(), p_T=fake(), algo=algo)
    a.update(over)
    return a


def call_validate(lib, a):
    return lib.kdn_validate_forward(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["c0"],
                                    a["mu"], a["variant"], a["dtype"], a["B"], a["T"], a["H"], a["dk"],
                                    a["dv"], a["S0"], a["p0"], a["o"], a["S_T"], a["p_T"], a["algo"])


def test_validate_forward_accepts_good_arguments(lib):
    f = Fake()
    for variant in (0, 1, 2, 3):
        for dtype in (0, 1):
            for dk in (64, 128):
                for dv in (64, 128):
                    assert call_validate(lib, fwd_args(f, variant=variant, dtype=dtype, dk=dk, dv=dv)) == 0
    assert call_validate(lib, fwd_args(f, B=0, q=None, o=None, S_T=None)) == 0  # empty batch
    assert call_validate(lib, fwd_args(f, T=0, q=None, k=None, v=None, o=None)) == 0  # empty sequence


@pytest.mark.parametrize("over,status", [
    (dict(q=None), kdn.KDN_ERR_NULL),
    (dict(o=None), kdn.KDN_ERR_NULL),
    (dict(S_T=None), kdn.KDN_ERR_NULL),
    (dict(p_T=None), kdn.KDN_ERR_NULL),
    (dict(c0=None), kdn.KDN_ERR_NULL),
    (dict(B=-1), kdn.KDN_ERR_SHAPE),
    (dict(T=-3), kdn.KDN_ERR_SHAPE),
    (dict(H=-1), kdn.KDN_ERR_SHAPE),
    (dict(B=1 << 20, H=1 << 12), kdn.KDN_ERR_SHAPE),
    (dict(dk=96), kdn.KDN_ERR_UNSUPPORTED),
    (dict(dv=32), kdn.KDN_ERR_UNSUPPORTED),
    (dict(dk=-64), kdn.KDN_ERR_SHAPE),
    (dict(variant=4), kdn.KDN_ERR_UNSUPPORTED),
    (dict(dtype=7), kdn.KDN_ERR_UNSUPPORTED),
    (dict(algo=9), kdn.KDN_ERR_UNSUPPORTED),
    (dict(mu=-1.0), kdn.KDN_ERR_VALUE),
    (dict(mu=float("nan")), kdn.KDN_ERR_VALUE),
    (dict(mu=float("inf")), kdn.KDN_ERR_VALUE),
])
def test_validate_forward_rejects(lib, over, status):
    f = Fake()
    assert call_validate(lib, fwd_args(f, **over)) == status
    assert lib.kdn_last_error()


def test_validate_forward_c0_optional_with_p0(lib):
    f = Fake()
    assert call_validate(lib, fwd_args(f, c0=None, p0=f())) == 0


def test_validate_forward_aliasing(lib):
    f = Fake()
    a = fwd_args(f)
    # S_T == S0 is allowed (continuation in place)
    s = f()
    assert call_validate(lib, dict(a, S0=s, S_T=s)) == 0
    # p_T == p0 is not
    p = f()
    assert call_validate(lib, dict(a, p0=p, p_T=p)) == kdn.KDN_ERR_ALIAS
    # o overlapping q
    assert call_validate(lib, dict(a, o=a["q"])) == kdn.KDN_ERR_ALIAS
    # S_T partially overlapping S0
    assert call_validate(lib, dict(a, S0=s, S_T=ctypes.c_void_p(s.value + 256))) == kdn.KDN_ERR_ALIAS
    # outputs overlapping each other
    assert call_validate(lib, dict(a, p_T=a["S_T"])) == kdn.KDN_ERR_ALIAS


def step_args(fake, N=4, H=2, dk=128, dv=128, variant=0, dtype=1, mu=128.0, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), omega=fake(), r=fake(), mu=mu, variant=variant,
             dtype=dtype, N=N, H=H, dk=dk, dv=dv, S=fake(), p=fake(), o=fake())
    a.update(over)
    return a


def call_validate_step(lib, a):
    return lib.kdn_validate_step(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["mu"],
                                 a["variant"], a["dtype"], a["N"], a["H"], a["dk"], a["dv"], a["S"],
                                 a["p"], a["o"])


@pytest.mark.parametrize("over,status", [
    (dict(), kdn.KDN_OK),
    (dict(N=0, q=None), kdn.KDN_OK),
    (dict(S=None), kdn.KDN_ERR_NULL),
    (dict(p=None), kdn.KDN_ERR_NULL),
    (dict(N=-1), kdn.KDN_ERR_SHAPE),
    (dict(dk=32), kdn.KDN_ERR_UNSUPPORTED),
    (dict(mu=-2.0), kdn.KDN_ERR_VALUE),
    (dict(variant=5), kdn.KDN_ERR_UNSUPPORTED),
    (dict(variant=2), kdn.KDN_OK),
])
def test_validate_step(lib, over, status):
    f = Fake()
    assert call_validate_step(lib, step_args(f, **over)) == status


def test_validate_step_aliasing(lib):
    f = Fake()
    a = step_args(f)
    assert call_validate_step(lib, dict(a, o=a["S"])) == kdn.KDN_ERR_ALIAS
    assert call_validate_step(lib, dict(a, p=a["k"])) == kdn.KDN_ERR_ALIAS


def test_launch_error_path_without_gpu(lib, monkeypatch):
    # KDN_FAULT=launch: validation passes, then the entry point reports a HIP
    # error instead of launching
    monkeypatch.setenv("KDN_FAULT", "launch")
    f = Fake()
    a = fwd_args(f)
    st = lib.kdn_forward(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["c0"], a["mu"],
                         a["variant"], a["dtype"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["S0"],
                         a["p0"], a["o"], a["S_T"], a["p_T"], None)
    assert st == kdn.KDN_ERR_HIP
    assert b"KDN_FAULT" in lib.kdn_last_error()
    s = step_args(f)
    st = lib.kdn_step(s["q"], s["k"], s["v"], s["alpha"], s["omega"], s["r"], s["mu"], s["variant"],
                      s["dtype"], s["N"], s["H"], s["dk"], s["dv"], s["S"], s["p"], s["o"], None)
    assert st == kdn.KDN_ERR_HIP
    # bad arguments are still reported as such, before the launch stage
    st = lib.kdn_forward(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["c0"], -1.0,
                         a["variant"], a["dtype"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["S0"],
                         a["p0"], a["o"], a["S_T"], a["p_T"], None)
    assert st == kdn.KDN_ERR_VALUE


def varlen_args(fake, N=3, total=40, H=2, dk=64, dv=64, variant=0, dtype=1, mu=64.0, algo=0, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), omega=fake(), r=fake(), cu=fake(), order=None, c0=fake(),
             mu=mu, variant=variant, dtype=dtype, N=N, total=total, H=H, dk=dk, dv=dv, S0=None, p0=None,
             o=fake(), S_T=fake(), p_T=fake(), algo=algo)
    a.update(over)
    return a


def call_validate_varlen(lib, a):
    return lib.kdn_validate_forward_varlen(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["cu"],
                                           a["order"], a["c0"], a["mu"], a["variant"], a["dtype"], a["N"], a["total"],
                                           a["H"], a["dk"], a["dv"], a["S0"], a["p0"], a["o"], a["S_T"],
                                           a["p_T"], a["algo"])


def test_validate_varlen_accepts_good_arguments(lib):
    f = Fake()
    for variant in (0, 1):
        for dtype in (0, 1):
            assert call_validate_varlen(lib, varlen_args(f, variant=variant, dtype=dtype)) == 0
    assert call_validate_varlen(lib, varlen_args(f, N=0, cu=None, q=None, S_T=None)) == 0  # no sequence
    # every sequence empty: no token input is read, the states are still written
    assert call_validate_varlen(lib, varlen_args(f, total=0, q=None, k=None, v=None, o=None)) == 0
    assert call_validate_varlen(lib, varlen_args(f, c0=None, p0=f())) == 0
    assert call_validate_varlen(lib, varlen_args(f, order=f())) == 0


@pytest.mark.parametrize("over,status", [
    (dict(cu=None), kdn.KDN_ERR_NULL),
    (dict(q=None), kdn.KDN_ERR_NULL),
    (dict(S_T=None), kdn.KDN_ERR_NULL),
    (dict(c0=None), kdn.KDN_ERR_NULL),
    (dict(N=-1), kdn.KDN_ERR_SHAPE),
    (dict(total=-5), kdn.KDN_ERR_SHAPE),
    (dict(H=-2), kdn.KDN_ERR_SHAPE),
    (dict(total=1 << 30, H=1 << 12), kdn.KDN_ERR_SHAPE),
    (dict(dk=96), kdn.KDN_ERR_UNSUPPORTED),
    (dict(algo=7), kdn.KDN_ERR_UNSUPPORTED),
    (dict(mu=-1.0), kdn.KDN_ERR_VALUE),
])
def test_validate_varlen_rejects(lib, over, status):
    f = Fake()
    assert call_validate_varlen(lib, varlen_args(f, **over)) == status
    assert lib.kdn_last_error()


def test_validate_varlen_aliasing(lib):
    f = Fake()
    a = varlen_args(f)
    assert call_validate_varlen(lib, dict(a, o=a["cu"])) == kdn.KDN_ERR_ALIAS  # the offsets are an input
    assert call_validate_varlen(lib, dict(a, p_T=a["cu"])) == kdn.KDN_ERR_ALIAS
    order = f()
    assert call_validate_varlen(lib, dict(a, order=order, o=order)) == kdn.KDN_ERR_ALIAS  # so is the order
    s = f()
    assert call_validate_varlen(lib, dict(a, S0=s, S_T=s)) == 0


def test_varlen_launch_error_path_without_gpu(lib, monkeypatch):
    monkeypatch.setenv("KDN_FAULT", "launch")
    f = Fake()
    a = varlen_args(f)
    args = [a[x] for x in ("q", "k", "v", "alpha", "omega", "r", "cu", "order", "c0", "mu", "variant", "dtype", "N",
                           "total", "H", "dk", "dv", "S0", "p0", "o", "S_T", "p_T")]
    assert lib.kdn_forward_varlen(*args, None, 0) == kdn.KDN_ERR_HIP
    args[6] = None  # no offsets: reported before the launch stage
    assert lib.kdn_forward_varlen(*args, None, 0) == kdn.KDN_ERR_NULL


def test_binding_raises_when_library_missing(tmp_path):
    saved = kdn._lib
    kdn._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            kdn.load_library(str(tmp_path / "nope.so"))
    finally:
        kdn._lib = saved


# ---------------------------------------------------------------------------
# kdn_backward
# ---------------------------------------------------------------------------

BWD_OUT = ("g_q", "g_k", "g_v", "g_alpha", "g_omega", "g_r", "g_S0", "g_p0", "g_c0")  # dq .. dc0


def bwd_args(fake, lib, B=2, T=40, H=2, dk=64, dv=64, variant=0, dtype=1, mu=64.0, **over):
    a = dict(q=fake(), k=fake(), v=fake(), alpha=fake(), omega=fake(), r=fake(), c0=fake(), mu=mu,
             variant=variant, dtype=dtype, B=B, T=T, H=H, dk=dk, dv=dv, S0=None, p0=None, dO=fake(),
             dS_T=None, dp_T=None, work=fake())
    for n in BWD_OUT:
        a[n] = fake()
    a["work_bytes"] = lib.kdn_backward_workspace_size(B, T, H, dk, dv)
    a.update(over)
    return a


def _bwd_list(a):
    return [a[n] for n in ("q", "k", "v", "alpha", "omega", "r", "c0", "mu", "variant", "dtype", "B", "T", "H",
                           "dk", "dv", "S0", "p0", "dO", "dS_T", "dp_T")] + [a[n] for n in BWD_OUT] + \
        [a["work"], a["work_bytes"]]


def call_validate_bwd(lib, a):
    return lib.kdn_validate_backward(*_bwd_list(a))


def test_backward_workspace_size_formula(lib):
    # every pair on the token path at once, then one int per (batch, head) pair (the chunked
    # path's range flags) rounded up to 256 bytes
    for B, T, H, dk, dv in ((2, 40, 3, 64, 128), (8, 4096, 16, 128, 128), (1, 1, 1, 128, 64)):
        want = B * H * token_pair_bytes(T, dk, dv) + r256(B * H * 4)
        assert lib.kdn_backward_workspace_size(B, T, H, dk, dv) == want
    assert lib.kdn_backward_workspace_size(0, 10, 2, 64, 64) == 0
    assert lib.kdn_backward_workspace_size(2, 0, 2, 64, 64) == 0


def test_backward_workspace_size_for(lib):
    # the diagonal bf16 form at dk, dv in {64, 128}: the chunked path's layout (with room for
    # one pair on the token path); everything else: the all-pairs size
    for B, T, H, dk, dv in ((2, 40, 3, 64, 128), (8, 4096, 16, 128, 128), (1, 1, 1, 128, 64),
                            (1, 65536, 16, 128, 128), (4, 1000, 2, 128, 64), (1, 4096, 1, 128, 128)):
        full = lib.kdn_backward_workspace_size(B, T, H, dk, dv)
        assert lib.kdn_backward_workspace_size_for(0, 1, B, T, H, dk, dv) == chunk_min_bytes(B, T, H, dk, dv)
        assert lib.kdn_backward_workspace_size_for(0, 1, B, T, H, dk, dv) <= full
        for variant, dtype in ((0, 0), (1, 1), (2, 1), (3, 1), (1, 0)):
            assert lib.kdn_backward_workspace_size_for(variant, dtype, B, T, H, dk, dv) == full
    # the diagonal bf16 backward at B=8, T=4096, H=16, d=128 within 1 GB (the all-pairs size is 4.2 GB)
    assert lib.kdn_backward_workspace_size_for(0, 1, 8, 4096, 16, 128, 128) == 873595392
    assert lib.kdn_backward_workspace_size_for(0, 1, 8, 4096, 16, 128, 128) < 10**9
    assert lib.kdn_backward_workspace_size_for(0, 1, 0, 10, 2, 64, 64) == 0
    assert lib.kdn_backward_workspace_size_for(0, 1, 2, 0, 2, 64, 64) == 0
    assert lib.kdn_backward_workspace_size_for(0, 1, 2, 10, 2, 96, 64) == lib.kdn_backward_workspace_size(
        2, 10, 2, 96, 64)


def test_validate_backward_workspace_for_variant(lib):
    # the smallest workspace each variant and dtype accepts, and one byte less
    f = Fake()
    for variant, dtype in ((0, 1), (0, 0), (1, 1)):
        need = lib.kdn_backward_workspace_size_for(variant, dtype, 2, 40, 2, 64, 64)
        assert call_validate_bwd(lib, bwd_args(f, lib, variant=variant, dtype=dtype, work_bytes=need)) == kdn.KDN_OK
        assert call_validate_bwd(lib, bwd_args(f, lib, variant=variant, dtype=dtype,
                                               work_bytes=need - 1)) == kdn.KDN_ERR_WORKSPACE


def test_validate_backward_accepts_good_arguments(lib):
    f = Fake()
    for variant in (0, 1, 2):
        for dtype in (0, 1):
            for dk in (64, 128):
                for dv in (64, 128):
                    assert call_validate_bwd(lib, bwd_args(f, lib, variant=variant, dtype=dtype, dk=dk, dv=dv)) == 0
    f = Fake()
    assert call_validate_bwd(lib, bwd_args(f, lib, dO=None, g_c0=None)) == 0  # cotangent and dc0 optional
    assert call_validate_bwd(lib, bwd_args(f, lib, S0=f(), p0=f(), c0=None, dS_T=f(), dp_T=f())) == 0
    assert call_validate_bwd(lib, bwd_args(f, lib, T=0, q=None, work=None)) == 0  # nothing to recompute


@pytest.mark.parametrize("over,status", [
    (dict(mu=-1.0), kdn.KDN_ERR_VALUE),
    (dict(dk=96), kdn.KDN_ERR_UNSUPPORTED),
    (dict(variant=4), kdn.KDN_ERR_UNSUPPORTED),
    (dict(T=-1), kdn.KDN_ERR_SHAPE),
    (dict(q=None), kdn.KDN_ERR_NULL),
    (dict(g_k=None), kdn.KDN_ERR_NULL),
    (dict(g_p0=None), kdn.KDN_ERR_NULL),
    (dict(c0=None), kdn.KDN_ERR_NULL),
    (dict(work=None), kdn.KDN_ERR_WORKSPACE),
    (dict(work_bytes=100), kdn.KDN_ERR_WORKSPACE),
    (dict(work=ctypes.c_void_p((1 << 44) + 8)), kdn.KDN_ERR_WORKSPACE),
    (dict(S0=ctypes.c_void_p((1 << 45) + 4)), kdn.KDN_ERR_UNSUPPORTED),
])
def test_validate_backward_rejects(lib, over, status):
    f = Fake()
    a = bwd_args(f, lib)
    assert call_validate_bwd(lib, dict(a, **over)) == status


def test_validate_backward_aliasing(lib):
    f = Fake()
    a = bwd_args(f, lib)
    assert call_validate_bwd(lib, dict(a, g_q=a["q"])) == kdn.KDN_ERR_ALIAS
    assert call_validate_bwd(lib, dict(a, g_v=a["dO"])) == kdn.KDN_ERR_ALIAS
    assert call_validate_bwd(lib, dict(a, g_S0=a["g_q"])) == kdn.KDN_ERR_ALIAS
    assert call_validate_bwd(lib, dict(a, work=a["g_r"])) == kdn.KDN_ERR_ALIAS


def test_backward_launch_error_path_without_gpu(lib, monkeypatch):
    monkeypatch.setenv("KDN_FAULT", "launch")
    f = Fake()
    a = bwd_args(f, lib)
    assert lib.kdn_backward(*_bwd_list(a), None) == kdn.KDN_ERR_HIP
    assert b"KDN_FAULT" in lib.kdn_last_error()
    assert lib.kdn_backward(*_bwd_list(dict(a, mu=float("nan"))), None) == kdn.KDN_ERR_VALUE


def test_grouped_noise_variant(lib):
    f = Fake()
    assert call_validate(lib, fwd_args(f, variant=3, dv=128)) == 0
    assert call_validate(lib, fwd_args(f, variant=4)) == kdn.KDN_ERR_UNSUPPORTED
    assert call_validate_bwd(lib, bwd_args(f, lib, variant=3, dv=128)) == 0
    assert call_validate_bwd(lib, bwd_args(f, lib, variant=4)) == kdn.KDN_ERR_UNSUPPORTED
    # r and p hold one entry per group of 64 value columns: an output placed
    # right after a single-group r overlaps the second group's entries
    a = fwd_args(f, variant=3, dk=64, dv=128, B=1, T=8, H=1)
    r_end = ctypes.c_void_p(a["r"].value + 8 * 2)  # bf16, 8 tokens x 1 group
    assert call_validate(lib, dict(a, o=r_end)) == kdn.KDN_ERR_ALIAS


def call_validate_gated(lib, a):
    return lib.kdn_validate_forward_gated(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["c0"],
                                          a["mu"], a["variant"], a["dtype"], a["B"], a["T"], a["H"], a["dk"],
                                          a["dv"], a["S0"], a["p0"], a["o"], a["S_T"], a["p_T"], a["algo"])


def test_validate_gated_forward(lib):
    # no gate step with grouped observation noise; the rest of the checks are
    # those of the plain forward
    f = Fake()
    for dtype in (0, 1):
        for algo in (0, 1, 2, 3, 4):
            assert call_validate_gated(lib, fwd_args(f, dtype=dtype, algo=algo)) == 0
    for variant in (1, 2):
        assert call_validate_gated(lib, fwd_args(f, variant=variant)) == 0
    assert call_validate_gated(lib, fwd_args(f, variant=3)) == kdn.KDN_ERR_UNSUPPORTED
    assert b"grouped" in lib.kdn_last_error()
    assert call_validate_gated(lib, fwd_args(f, q=None)) == kdn.KDN_ERR_NULL
    assert call_validate_gated(lib, fwd_args(f, dk=96)) == kdn.KDN_ERR_UNSUPPORTED
    assert call_validate_gated(lib, fwd_args(f, mu=-1.0)) == kdn.KDN_ERR_VALUE
    assert call_validate_gated(lib, fwd_args(f, B=0, q=None, o=None, S_T=None)) == 0


def test_gated_serving_entry_points_refuse_grouped_noise_before_any_launch(lib):
    # argument errors return before anything touches the device
    f = Fake()
    assert lib.kdn_step_gated(f(), f(), f(), f(), f(), f(), 128.0, 3, 1, 2, 3, 128, 128, f(), f(), f(),
                              None) == kdn.KDN_ERR_UNSUPPORTED
    assert lib.kdn_step_gated(None, f(), f(), f(), f(), f(), 128.0, 0, 1, 2, 3, 128, 128, f(), f(), f(),
                              None) == kdn.KDN_ERR_NULL
    assert lib.kdn_forward_varlen_gated(f(), f(), f(), f(), f(), f(), f(), None, f(), 128.0, 3, 1, 2, 10, 3,
                                        128, 128, None, None, f(), f(), f(), None, 0) == kdn.KDN_ERR_UNSUPPORTED
    assert lib.kdn_step_gated(f(), f(), f(), f(), f(), f(), 128.0, 0, 1, 0, 3, 128, 128, f(), f(), f(),
                              None) == kdn.KDN_OK  # empty batch: nothing to launch


def test_gated_backward_workspace_size_formula(lib):
    # the adjoint's workspace, then fp32 q, k, v, dO, alpha, omega, r, each
    # rounded up to 256 bytes; none for grouped noise
    base = kdn.backward_workspace_size(2, 33, 2, 128, 64)
    r256 = lambda n: (n + 255) // 256 * 256
    toks = 2 * 33 * 2
    assert kdn.backward_gated_workspace_size(2, 33, 2, 128, 64) == (
        r256(base) + 2 * r256(toks * 128 * 4) + 2 * r256(toks * 64 * 4) + 2 * r256(toks * 128 * 4) + r256(toks * 4))
    assert kdn.backward_gated_workspace_size(2, 33, 2, 128, 64, "isotropic") == (
        r256(base) + 2 * r256(toks * 128 * 4) + 2 * r256(toks * 64 * 4) + 3 * r256(toks * 4))
    assert kdn.backward_gated_workspace_size(2, 33, 2, 128, 64, "grouped") == 0
    # the smallest: the adjoint's smallest workspace for the variant and dtype, the same copies
    copies = 2 * r256(toks * 128 * 4) + 2 * r256(toks * 64 * 4) + 2 * r256(toks * 128 * 4) + r256(toks * 4)
    for dtype in (0, 1):
        assert lib.kdn_backward_gated_workspace_size_for(0, dtype, 2, 33, 2, 128, 64) == (
            r256(lib.kdn_backward_workspace_size_for(0, dtype, 2, 33, 2, 128, 64)) + copies)
    big = lib.kdn_backward_gated_workspace_size_for(0, 1, 8, 4096, 16, 128, 128)
    assert big == r256(chunk_min_bytes(8, 4096, 16, 128, 128)) + 8 * 4096 * 16 * 4 * (6 * 128 + 1)
    assert lib.kdn_backward_gated_workspace_size_for(3, 1, 2, 33, 2, 128, 64) == 0
    assert kdn.backward_gated_workspace_size(0, 33, 2, 128, 64) == 0


def test_noalloc_backward_host_checks_without_gpu(lib, monkeypatch):
    # kdn_backward_noalloc: sizes whose workspace exceeds the static scratch are
    # refused before any device access; with the launch fault hook the call
    # reports the launch error (its remaining checks and the scratch need a GPU)
    f = Fake()
    big = bwd_args(f, lib, B=1, T=8192, H=16, dk=128, dv=128)
    assert lib.kdn_backward_workspace_size_for(0, 1, 1, 8192, 16, 128, 128) > kdn.NOALLOC_SCRATCH_BYTES
    noalloc = lambda a: lib.kdn_backward_noalloc(*_bwd_list(a)[:-2], None)
    assert noalloc(big) == kdn.KDN_ERR_WORKSPACE
    assert b"static scratch" in lib.kdn_last_error()
    assert noalloc(bwd_args(f, lib, mu=-1.0)) == kdn.KDN_ERR_VALUE
    assert noalloc(bwd_args(f, lib, dk=96)) == kdn.KDN_ERR_UNSUPPORTED
    monkeypatch.setenv("KDN_FAULT", "launch")
    assert noalloc(bwd_args(f, lib)) == kdn.KDN_ERR_HIP
    assert b"KDN_FAULT" in lib.kdn_last_error()


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define KDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == kdn.NOALLOC_SCRATCH_BYTES


# ---------------------------------------------------------------------------
# kdn_forward_split: validation and workspace sizes (host only)
# ---------------------------------------------------------------------------

def call_validate_split(lib, a, segments, ws, ws_bytes):
    return lib.kdn_validate_forward_split(a["q"], a["k"], a["v"], a["alpha"], a["omega"], a["r"], a["c0"],
                                          a["mu"], a["variant"], a["dtype"], a["B"], a["T"], a["H"], a["dk"],
                                          a["dv"], a["S0"], a["p0"], a["o"], a["S_T"], a["p_T"], segments, ws,
                                          ws_bytes)


def test_split_workspace_size(lib):
    size = lib.kdn_forward_split_workspace_size
    # no split: one segment asked for, or a sequence too short to cut
    assert size(1, 8192, 2, 128, 128, 1) == 0
    assert size(1, 40, 2, 128, 128, 4) == 0
    # four segments of 2048 tokens (sub-segments of 256), B=1, H=2,
    # d_k=d_v=128: sub-segment and
    # segment products, identity-column outputs (bf16), end states [v | I]
    # (fp32) and start states (bf16), each region rounded up to 256 bytes
    units, nseg, nsub, T = 2, 4, 8, 8192
    r256 = lambda x: (x + 255) // 256 * 256
    want = (r256(units * nseg * nsub * 128 * 16) + r256(units * nseg * 128 * 16) + r256(T * 2 * 128 * 2)
            + r256(units * nseg * 128 * 256 * 4) + r256(units * nseg * 128 * 128 * 2))
    assert size(1, T, 2, 128, 128, 4) == want
    assert size(0, T, 2, 128, 128, 4) == 0 and size(1, T, 2, 96, 128, 4) == 0 and size(1, T, 2, 128, 128, -1) == 0


def test_split_segments(lib):
    seg = lib.kdn_forward_split_segments
    assert seg(1, 8192, 2, 128, 128, 4) == 4
    assert seg(1, 8192, 2, 128, 128, 1) == 1
    assert seg(1, 1000, 2, 128, 128, 3) == 3  # segments of 352, 352 and 296 tokens
    assert seg(1, 40, 2, 128, 128, 4) == 1    # too short to cut
    assert seg(0, 8192, 2, 128, 128, 4) == 0 and seg(1, 8192, 2, 128, 128, -1) == 0
    # chosen: as many segments as fill the compute units (here at least the
    # 256 of the fallback when no device is visible, or the device's own)
    assert seg(8, 4096, 16, 128, 128, 0) == 1  # B x H already fills the device
    assert seg(1, 65536, 16, 128, 128, 0) >= 2


def test_validate_split(lib):
    f = Fake()
    a = fwd_args(f, B=1, T=8192, H=2, dk=128, dv=128)
    need = lib.kdn_forward_split_workspace_size(1, 8192, 2, 128, 128, 4)
    ws = f()
    assert need > 0
    assert call_validate_split(lib, a, 4, ws, need) == 0
    assert call_validate_split(lib, a, 1, None, 0) == 0  # no split: no workspace needed
    assert call_validate_split(lib, a, 4, None, need) == kdn.KDN_ERR_WORKSPACE
    assert call_validate_split(lib, a, 4, ws, need - 1) == kdn.KDN_ERR_WORKSPACE
    assert call_validate_split(lib, a, 4, ctypes.c_void_p(ws.value + 8), need) == kdn.KDN_ERR_WORKSPACE
    assert call_validate_split(lib, a, 4, a["o"], need) == kdn.KDN_ERR_ALIAS
    assert call_validate_split(lib, a, -1, ws, need) == kdn.KDN_ERR_VALUE
    assert call_validate_split(lib, dict(a, variant=1), 4, ws, need) == kdn.KDN_ERR_UNSUPPORTED
    assert call_validate_split(lib, dict(a, dtype=0), 4, ws, need) == kdn.KDN_ERR_UNSUPPORTED
    assert call_validate_split(lib, dict(a, q=None), 4, ws, need) == kdn.KDN_ERR_NULL
