"""Pins for the fp64 oracle's backward pass (the reverse-mode adjoint of the
KDN recurrence: "Kalman Delta Networks: Uncertainty-aware Associative
Memory", summary page, method steps 2-5, and its closing sentence for the
isotropic forms).

The adjoint is pinned to the forward oracle (itself pinned in
test_oracle_pins.py) by central finite differences in fp64: every element
of every input, of the initial state and of c0, on tiny problems.  A dropped
term, a wrong sign or a transposed operand anywhere in the adjoint changes
some derivative by far more than the differencing error.
"""
import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl

FWD = {"diagonal": oracle.forward_diag, "isotropic": oracle.forward_iso, "isochannel": oracle.forward_isoc,
       "grouped": oracle.forward_grouped}
TOKEN = ("q", "k", "v", "alpha", "omega", "r")


def _case(variant, with_state, seed, B=2, T=6, H=2, dk=4, dv=3, omega_loc=-1.0, mu=None, rgroups=1):
    w = wl.Workload("fd", variant, "f32", B, T, H, dk, dv, float(dk if mu is None else mu), "uniform",
                    seed, omega_loc=omega_loc, rgroups=rgroups)
    x = {n: np.asarray(a, np.float64) for n, a in wl.forward_inputs(w).items()}
    ct = wl.backward_cotangents(w, with_state=True)
    st = wl.decode_state(w) if with_state else {"S0": None, "p0": None}
    return w, x, ct, st


def _loss(w, x, ct, st):
    out = FWD[w.variant](**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, S0=st["S0"], p0=st["p0"])
    return (np.sum(out["o"] * ct["dO"]) + np.sum(out["S"] * ct["dS_T"]) + np.sum(out["p"] * ct["dp_T"]))


def _fd(w, x, ct, st, holder, name, eps=1e-6):
    arr = holder[name]
    g = np.zeros(arr.shape)
    flat, gflat = arr.reshape(-1), g.reshape(-1)
    for e in range(flat.size):
        base = flat[e]
        h = eps * max(1.0, abs(base))
        flat[e] = base + h
        lp = _loss(w, x, ct, st)
        flat[e] = base - h
        lm = _loss(w, x, ct, st)
        flat[e] = base
        gflat[e] = (lp - lm) / (2 * h)
    return g


def _check(g, fd, name):
    scale = max(np.max(np.abs(fd)), 1e-12)
    err = np.max(np.abs(g - fd)) / scale
    assert err < 1e-6, (name, err)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
@pytest.mark.parametrize("with_state", [True, False])
def test_backward_matches_finite_differences(variant, with_state):
    w, x, ct, st = _case(variant, with_state, seed=31 + with_state)
    if with_state:
        st = {n: np.asarray(a, np.float64) for n, a in st.items()}
    g = oracle.backward(**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                        dp_T=ct["dp_T"], S0=st["S0"], p0=st["p0"], variant=variant)
    for name in TOKEN:
        _check(g["d" + name], _fd(w, x, ct, st, x, name), name)
    if with_state:
        _check(g["dS0"], _fd(w, x, ct, st, st, "S0"), "S0")
        _check(g["dp0"], _fd(w, x, ct, st, st, "p0"), "p0")
    else:
        # p_0 = c0[h] on every channel: dc0 is the derivative with respect to c0
        _check(g["dc0"], _fd(w, x, ct, st, x, "c0"), "c0")
        np.testing.assert_allclose(g["dc0"], g["dp0"].reshape(w.B, w.H, -1).sum(axis=(0, 2)), rtol=1e-12)


@pytest.mark.parametrize("with_state", [True, False])
def test_grouped_noise_backward_matches_finite_differences(with_state):
    w, x, ct, st = _case("grouped", with_state, seed=41 + with_state, dv=4, rgroups=2)
    if with_state:
        st = {n: np.asarray(a, np.float64) for n, a in st.items()}
    g = oracle.backward(**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                        dp_T=ct["dp_T"], S0=st["S0"], p0=st["p0"], variant="grouped")
    for name in TOKEN:
        _check(g["d" + name], _fd(w, x, ct, st, x, name), name)
    if with_state:
        _check(g["dS0"], _fd(w, x, ct, st, st, "S0"), "S0")
        _check(g["dp0"], _fd(w, x, ct, st, st, "p0"), "p0")
    else:
        _check(g["dc0"], _fd(w, x, ct, st, x, "c0"), "c0")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_backward_strong_writes_and_slow_decay(variant):
    """Large process noise (gains near 1) and several chunks' worth of tokens
    with slow decay: the regime where a wrong gain derivative shows most."""
    w, x, ct, st = _case(variant, False, seed=57, B=1, T=12, H=1, dk=4, dv=2, omega_loc=1.5)
    g = oracle.backward(**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                        dp_T=ct["dp_T"], variant=variant)
    for name in TOKEN:
        _check(g["d" + name], _fd(w, x, ct, st, x, name), name)


def test_backward_zero_cotangents_give_zero_gradients():
    w, x, ct, st = _case("diagonal", False, seed=3)
    g = oracle.backward(**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, variant="diagonal")
    for val in g.values():
        assert np.count_nonzero(val) == 0


def test_uncertainty_gradient_closed_form_without_dynamics():
    """With alpha = 1, omega = 0 and only dp_T given, p_T = 1/(1/p0 + mu sum k^2/r)
    (precision additivity): its derivative with respect to p0 is
    (p_T/p0)^2, a closed form independent of the adjoint's code."""
    w, x, ct, st = _case("diagonal", True, seed=9, B=1, T=5, H=1, dk=3, dv=2)
    x["alpha"][:] = 1.0
    x["omega"][:] = 0.0
    p0 = np.asarray(st["p0"], np.float64)
    dp_T = np.ones_like(p0)
    g = oracle.backward(**{n: x[n] for n in TOKEN}, c0=x["c0"], mu=w.mu, dp_T=dp_T, S0=st["S0"], p0=p0)
    prec = 1.0 / p0 + w.mu * np.sum(x["k"][0, :, 0, :] ** 2 / x["r"][0, :, 0, None], axis=0)[None, None, :]
    pT = 1.0 / prec
    np.testing.assert_allclose(g["dp0"], (pT / p0) ** 2, rtol=1e-12)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic", "isochannel"])
def test_gated_backward_matches_finite_differences_of_the_gated_forward(variant):
    # gradients with respect to the gate pre-activations, against central
    # differences of oracle.forward_gated (the gate step of the summary page,
    # method step 1)
    w, x, ct, _ = _case(variant, False, seed=51)
    z = {n: np.asarray(a, np.float64) for n, a in wl.gated_inputs(w).items()}
    names = ("q", "k", "v", "z_alpha", "z_omega", "z_r")

    def loss():
        out = oracle.forward_gated(**{n: z[n] for n in names}, c0=z["c0"], mu=w.mu, variant=variant)
        return np.sum(out["o"] * ct["dO"]) + np.sum(out["S"] * ct["dS_T"]) + np.sum(out["p"] * ct["dp_T"])

    g = oracle.backward_gated(**{n: z[n] for n in names}, c0=z["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                              dp_T=ct["dp_T"], variant=variant)
    for name in ("z_alpha", "z_omega", "z_r", "k", "q"):
        arr = z[name]
        fd = np.zeros(arr.shape)
        flat, gflat = arr.reshape(-1), fd.reshape(-1)
        for e in range(flat.size):
            base = flat[e]
            h = 1e-6 * max(1.0, abs(base))
            flat[e] = base + h
            lp = loss()
            flat[e] = base - h
            lm = loss()
            flat[e] = base
            gflat[e] = (lp - lm) / (2 * h)
        _check(g["d" + name], fd, name)


def test_l2norm_backward_matches_finite_differences():
    # the cotangent of the raw rows through the normalisation, against
    # central differences of <l2norm(x), c>, including a row below the floor
    rng = np.random.default_rng(61)
    x = rng.standard_normal((4, 3, 8))
    x[1, 2] *= 1e-9
    c = rng.standard_normal(x.shape)
    g = oracle.l2norm_backward(x, c)
    fd = np.zeros(x.shape)
    flat, gf = x.reshape(-1), fd.reshape(-1)
    for e in range(flat.size):
        base = flat[e]
        h = 1e-7 * max(1e-6, abs(base))
        flat[e] = base + h
        lp = np.sum(oracle.l2norm(x) * c)
        flat[e] = base - h
        lm = np.sum(oracle.l2norm(x) * c)
        flat[e] = base
        gf[e] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-6 * np.max(np.abs(fd)))


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_gated_backward_q_k_gradients_are_orthogonal_to_the_rows(variant):
    # the loss depends on q and k only through q / |q| and k / |k|, so the
    # gradient of each row is orthogonal to the row
    w, x, ct, _ = _case(variant, False, seed=52)
    z = {n: np.asarray(a, np.float64) for n, a in wl.gated_inputs(w).items()}
    names = ("q", "k", "v", "z_alpha", "z_omega", "z_r")
    g = oracle.backward_gated(**{n: z[n] for n in names}, c0=z["c0"], mu=w.mu, dO=ct["dO"], dS_T=ct["dS_T"],
                              dp_T=ct["dp_T"], variant=variant)
    for n in ("q", "k"):
        dot = np.sum(g["d" + n] * z[n], axis=-1)
        scale = np.max(np.abs(g["d" + n])) * np.max(np.linalg.norm(z[n], axis=-1))
        assert np.max(np.abs(dot)) < 1e-12 * scale, n
