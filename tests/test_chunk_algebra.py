"""CPU model of the chunked kernel's blocked algebra (design check, no GPU).

The chunked forward rewrites 32 tokens of the diagonal KDN recurrence
("Kalman Delta Networks: Uncertainty-aware Associative Memory", summary page,
method steps 2-5) as matrix products.  Inside a chunk the decay between token
s and a later token t is the product of alpha over s+1..t; the kernel factors
it as rho_t / rho_s with every rho referenced to the chunk's midpoint (the
boundary between tokens 15 and 16):

  rho_t = g_t / g_15 (t <= 15, >= 1),  rho_t = prod_{16<=u<=t} alpha_u (t >= 16, <= 1)
  Kt = k rho, Qt = q rho, Kh = p_hat k / rho
  Sg = diag(g_15) S_c
  M  = diag(r) + tril(Kt Kh^T),  R = V - Kt Sg,  Dn = M^-1 R
  O  = Qt Sg + tril(Qt Kh^T) Dn,  S_{c+1} = diag(gb_31) (Sg + Kh^T Dn)

so no operand carries more than one half-chunk's decay.  A chunk whose
half-chunk decay (g_15 or gb_31, on any channel) falls below 2^-96 is outside
the fast form's range: the workgroup finishes the sequence with the token
recurrence from that chunk on.  These tests model exactly that, in fp64 (the
algebra is an identity) and in fp32 with bf16 matrix operands (the ranges),
and compare with the fp64 oracle.  They also show that the chunk-start
reference (Kh = p_hat k / g_t over all 32 tokens) overflows fp32 where the
midpoint reference does not.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from kalman_delta_network_amd import workloads as wl

L = 32
THETA = 96  # the fast form needs every half-chunk decay >= 2^-THETA


def _bf(x, emulate):
    return wl.round_bf16(np.asarray(x, np.float32)).astype(np.float64) if emulate else x


def _ft(x, emulate):
    """fp32 rounding of an accumulator (emulate) or nothing (fp64 model).  The
    upper triangles of the chunk products (t < s, discarded by tril) may
    exceed the fp32 range; that overflow is expected."""
    if not emulate:
        return x
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float64)


def chunk_model(q, k, v, alpha, omega, r, c0, mu, emulate=False):
    """One (batch, head) pair: q, k, alpha, omega [T, dk]; v [T, dv]; r [T].
    Returns o, S_T, p_T, the first chunk outside the fast form's range (or
    None) and the largest |operand| the fast form produced."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv))
    p = np.full(dk, float(c0))
    o = np.zeros((T, dv))
    big = 0.0
    nch = (T + L - 1) // L
    for c in range(nch):
        t0, t1 = c * L, min(T, (c + 1) * L)
        n = t1 - t0
        # chain: uncertainty recurrence (sequential per channel) and decays
        ph = np.zeros((n, dk))
        pe = p.copy()
        for j in range(n):
            ph[j] = alpha[t0 + j] ** 2 * pe + omega[t0 + j]
            pe = ph[j] / (1.0 + (mu / r[t0 + j]) * k[t0 + j] ** 2 * ph[j])
        a = np.ones((L, dk))
        a[:n] = alpha[t0:t1]
        g = np.cumprod(a[:16], axis=0)              # g_t, t <= 15
        gb = np.cumprod(a[16:], axis=0)             # prod over 16..t, t >= 16
        g15, gb31 = g[15], gb[-1]
        if np.min(g15) < 2.0 ** -THETA or np.min(gb31) < 2.0 ** -THETA:
            # outside the fast form: token recurrence from this chunk on
            rest = {nm: x[None, t0:, None] for nm, x in (("q", q), ("k", k), ("v", v), ("alpha", alpha),
                                                          ("omega", omega))}
            res = oracle.forward_diag(**rest, r=r[None, t0:, None], c0=np.array([1.0]), mu=mu,
                                      S0=S[None, None], p0=p[None, None])
            o[t0:] = res["o"][0, :, 0]
            return o, res["S"][0, 0], res["p"][0, 0], c, big
        rho = np.concatenate([g / g15, gb])[:n]
        kap = ph * k[t0:t1]
        Kt = _bf(k[t0:t1] * rho, emulate)
        Qt = _bf(q[t0:t1] * rho, emulate)
        Kh = _bf(kap / rho, emulate)
        big = max(big, float(np.max(np.abs(np.concatenate([Kt, Qt, Kh])))))
        Sg = _ft(g15[:, None] * S, emulate)
        M = np.diag(r[t0:t1]) + np.tril(_ft(Kt @ Kh.T, emulate))
        R = _ft(v[t0:t1] - Kt @ _bf(Sg, emulate), emulate)
        Dn = np.linalg.solve(M, R)
        QK = np.tril(_ft(Qt @ Kh.T, emulate))
        o[t0:t1] = _ft(Qt @ _bf(Sg, emulate) + _bf(QK, emulate) @ _bf(Dn, emulate), emulate)
        S = _ft(gb31[:, None] * _ft(Sg + Kh.T @ _bf(Dn, emulate), emulate), emulate)
        p = pe
    return o, S, p, None, big


def _inputs(T, dk, dv, alpha_loc, seed, alpha_const=None, const_chunk=None):
    w = wl.Workload("model", "diagonal", "bf16", 1, T, 1, dk, dv, float(dk), "one", seed, alpha_loc=alpha_loc,
                    omega_loc=-2.0)
    x = wl.forward_inputs(w)
    x = {n: (x[n][0, :, 0].astype(np.float64) if n != "c0" else x[n]) for n in x}
    if alpha_const is not None:
        lo, hi = const_chunk * L, (const_chunk + 1) * L
        x["alpha"][lo:hi] = float(wl.round_bf16(np.array([alpha_const], np.float32))[0])
    return x, w.mu


def _ref(x, mu):
    res = oracle.forward_diag(**{n: x[n][None, :, None] for n in ("q", "k", "v", "alpha", "omega")},
                              r=x["r"][None, :, None], c0=x["c0"][:1], mu=mu)
    return res["o"][0, :, 0], res["S"][0, 0], res["p"][0, 0]


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("alpha_loc", [2.0, 0.0, -3.0])
def test_midpoint_form_is_the_recurrence(alpha_loc):
    # fp64: the blocked algebra equals the token recurrence (an identity)
    x, mu = _inputs(200, 64, 64, alpha_loc, 31)
    o, S, p, bad, _ = chunk_model(x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], 1.0, mu)
    assert bad is None
    ro, rS, rp = _ref(x, mu)
    assert _rel(o, ro) < 1e-10 and _rel(S, rS) < 1e-10 and _rel(p, rp) < 1e-12


@pytest.mark.parametrize("alpha_const", [1e-3, 1e-6])
def test_tiny_decay_switches_to_the_recurrence(alpha_const):
    # a full chunk at alpha = 1e-3 or 1e-6 is outside the fast form's range;
    # chunks before it use the fast form, the rest the token recurrence
    x, mu = _inputs(150, 64, 64, 2.0, 32, alpha_const=alpha_const, const_chunk=2)
    o, S, p, bad, _ = chunk_model(x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], 1.0, mu)
    assert bad == 2
    ro, rS, rp = _ref(x, mu)
    assert _rel(o, ro) < 1e-10 and _rel(S, rS) < 1e-10 and _rel(p, rp) < 1e-12


@pytest.mark.parametrize("alpha_loc", [2.0, -3.0])
def test_midpoint_form_in_fp32_with_bf16_operands(alpha_loc):
    # the kernel's precisions: every operand finite and below 2^127, the
    # outputs within the bf16 tolerance of the fp64 recurrence.
    # alpha_loc = -3: alpha ~ sigmoid(N(-3, 0.5)) ~ 0.05, a 16-token decay of
    # about 2^-70 (inside the fast form), a 32-token decay of about 2^-140
    x, mu = _inputs(256, 128, 128, alpha_loc, 33)
    o, S, p, bad, big = chunk_model(x["q"], x["k"], x["v"], x["alpha"], x["omega"], x["r"], 1.0, mu, emulate=True)
    assert bad is None and np.isfinite(big) and big < 2.0 ** 127
    ro, rS, rp = _ref(x, mu)
    assert _rel(o, ro) < 2e-2 and _rel(S, rS) < 2e-2 and _rel(p, rp) < 1e-6


def test_chunk_start_reference_overflows_where_midpoint_does_not():
    # alpha ~ sigmoid(N(-3, 0.5)): p_hat k / g_t over a whole chunk exceeds the
    # fp32 (and bf16) range, the midpoint-referenced operands stay below 2^96
    x, mu = _inputs(256, 128, 128, -3.0, 34)
    a = x["alpha"][:L]
    g = np.cumprod(a, axis=0)
    assert np.max(1.0 / g) > np.finfo(np.float32).max
    g15 = g[15]
    rho = np.concatenate([g[:16] / g15, np.cumprod(a[16:], axis=0)])
    assert np.max(rho) < 2.0 ** THETA and np.max(1.0 / rho) < 2.0 ** THETA
