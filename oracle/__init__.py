"""fp64 CPU oracle for the Kalman Delta Network recurrence.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code
with the HIP library (kalman_delta_network_amd) and the library never calls
it.

* ``forward_diag`` / ``forward_iso`` / ``forward_isoc`` and the ``step_*``
  decode steps wrap the
  sequential fp64 recurrence in ``kdn_oracle.c`` ("Kalman Delta Networks:
  Uncertainty-aware Associative Memory", summary page, section on the
  method steps, steps 2-5, and its closing sentence for the isotropic
  variant).
* ``forward_varlen`` runs packed variable-length batches through the same
  recurrence, one sequence at a time.
* ``forward_grouped`` is the diagonal recurrence with block-diagonal
  observation noise over groups of value columns (one per group).
* ``backward`` is the reverse-mode adjoint of the same recurrence (the
  gradients a training step needs), pinned by central finite differences of
  the forward.
* ``gates`` and ``forward_gated``: the gate step that precedes the
  recurrence (same summary page, method step 1): decay alpha = sigmoid(z),
  process noise omega = softplus(z) and observation noise
  r = r_min + softplus(z) with r_min = 0.01, from their pre-activations.
* ``dense`` holds the brute-force dense-covariance filter (Bayesian Layer
  page, section 2.2, Proposition 1) used to pin the oracle.

Every function here is pinned by CPU tests in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB = os.path.join(_HERE, "libkdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP over independent heads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        fwd = [I, I, I, I, I, P, P, P, P, P, P, P, D, P, P, P, P, P, P, P, P]
        for name in ("kdn_oracle_forward_diag", "kdn_oracle_forward_iso", "kdn_oracle_forward_isoc"):
            fn = getattr(lib, name)
            fn.argtypes = fwd
            fn.restype = I
        stp = [I, I, I, I, P, P, P, P, P, P, D, P, P, P]
        for name in ("kdn_oracle_step_diag", "kdn_oracle_step_iso", "kdn_oracle_step_isoc"):
            fn = getattr(lib, name)
            fn.argtypes = stp
            fn.restype = I
        lib.kdn_oracle_backward.argtypes = [I, I, I, I, I, I] + [P] * 7 + [D] + [P] * 14
        lib.kdn_oracle_backward.restype = I
        lib.kdn_oracle_num_threads.restype = I
        lib.kdn_oracle_set_num_threads.argtypes = [I]
        lib.kdn_oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().kdn_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Use n threads in the oracle's OpenMP loops from now on."""
    _load().kdn_oracle_set_num_threads(int(n))


def _in(x):
    """Token inputs as contiguous float64 (bf16 / fp32 values widen exactly)."""
    return np.ascontiguousarray(x, dtype=np.float64)


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _forward(name, q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None, trace=False):
    q, k, v, alpha, omega, r = (_in(x) for x in (q, k, v, alpha, omega, r))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    iso = name.endswith(("iso", "isoc"))
    c0 = _in(np.broadcast_to(np.asarray(c0, np.float64), (H,)))
    S0, p0 = _f64(S0), _f64(p0)
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    p_T = np.zeros((B, H) if iso else (B, H, dk))
    tr = None
    if trace:
        tshape = (B, T, H) if iso else (B, T, H, dk)
        tr = {"p_hat": np.zeros(tshape), "kappa": np.zeros((B, T, H, dk)), "p": np.zeros(tshape)}
    rc = getattr(_load(), name)(
        B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0),
        float(mu), _ptr(S0), _ptr(p0), _ptr(o), _ptr(S_T), _ptr(p_T),
        _ptr(tr["p_hat"]) if tr else None, _ptr(tr["kappa"]) if tr else None,
        _ptr(tr["p"]) if tr else None)
    if rc != 0:
        raise ValueError(f"{name}: bad arguments (rc={rc})")
    out = {"o": o, "S": S_T, "p": p_T}
    if tr:
        out.update({"trace_" + key: val for key, val in tr.items()})
    return out


def forward_diag(q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None, trace=False):
    """Diagonal KDN forward.  Shapes: q,k,alpha,omega [B,T,H,dk]; v [B,T,H,dv];
    r [B,T,H]; c0 [H] (or scalar); S0 [B,H,dk,dv]; p0 [B,H,dk].
    Returns dict o [B,T,H,dv], S [B,H,dk,dv], p [B,H,dk] (+ traces)."""
    return _forward("kdn_oracle_forward_diag", q, k, v, alpha, omega, r, c0, mu, S0, p0, trace)


def forward_iso(q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None, trace=False):
    """Isotropic KDN forward.  alpha, omega, r [B,T,H]; p0 / returned p [B,H]."""
    return _forward("kdn_oracle_forward_iso", q, k, v, alpha, omega, r, c0, mu, S0, p0, trace)


def forward_varlen(q, k, v, alpha, omega, r, c0, mu, cu_seqlens, variant="diagonal", S0=None, p0=None):
    """Packed variable-length forward: sequence n is the token rows
    cu_seqlens[n] .. cu_seqlens[n+1]-1 of the [total,H,*] inputs, run from its
    own initial state (S0[n], p0[n]; zero memory and c0 when absent) by
    forward_diag / forward_iso.  The recurrence is per sequence; packing only
    decides which rows belong to which sequence.
    Returns o [total,H,dv], S [N,H,dk,dv], p [N,H,dk] (isotropic [N,H])."""
    fn = {"diagonal": forward_diag, "isotropic": forward_iso, "isochannel": forward_isoc,
          "grouped": forward_grouped}[variant]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or len(cu) < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != len(q):
        raise ValueError("cu_seqlens must rise from 0 to the number of token rows")
    N = len(cu) - 1
    total, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = np.zeros((total, H, dv))
    S = np.zeros((N, H, dk, dv))
    pshape = {"diagonal": (N, H, dk), "grouped": (N, H, np.shape(r)[-1], dk)}.get(variant, (N, H))
    p = np.zeros(pshape)  # isotropic forms: one scalar per head
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        out = fn(*(np.asarray(x)[None, a:b] for x in (q, k, v, alpha, omega, r)), c0, mu,
                 None if S0 is None else np.asarray(S0)[n:n + 1], None if p0 is None else np.asarray(p0)[n:n + 1])
        o[a:b] = out["o"][0]
        S[n] = out["S"][0]
        p[n] = out["p"][0]
    return {"o": o, "S": S, "p": p}


def forward_grouped(q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None):
    """Diagonal KDN with grouped observation noise ("Memory by Design:
    Probabilistic Sequence Layers", section on per-column and grouped
    observation noise): the noise covariance is block diagonal over G groups
    of d_v / G value columns, diag[r_1 I, ..., r_G I], so each group keeps its
    own key-space uncertainty and gain.  The groups share q, k, alpha, omega
    and are otherwise independent, so each is the diagonal recurrence
    (forward_diag) on its value columns with its own r and p.
    Shapes as forward_diag except r [B,T,H,G], p0 / returned p [B,H,G,dk]."""
    r = np.asarray(r)
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    G = r.shape[-1]
    if dv % G:
        raise ValueError("d_v must be a multiple of the number of groups")
    gw = dv // G
    o = np.zeros((B, T, H, dv))
    S = np.zeros((B, H, dk, dv))
    p = np.zeros((B, H, G, dk))
    for g in range(G):
        cols = slice(g * gw, (g + 1) * gw)
        out = forward_diag(q, k, np.asarray(v)[..., cols], alpha, omega, r[..., g], c0, mu,
                           None if S0 is None else np.asarray(S0)[..., cols],
                           None if p0 is None else np.asarray(p0)[:, :, g])
        o[..., cols] = out["o"]
        S[..., cols] = out["S"]
        p[:, :, g] = out["p"]
    return {"o": o, "S": S, "p": p}


def forward_isoc(q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None, trace=False):
    """Isotropic KDN with per-channel decay: alpha [B,T,H,dk] (the memory
    decays by diag(alpha), the uncertainty scalar by mean_i alpha_i^2);
    omega, r [B,T,H]; p0 / returned p [B,H]."""
    return _forward("kdn_oracle_forward_isoc", q, k, v, alpha, omega, r, c0, mu, S0, p0, trace)


def _step(name, q, k, v, alpha, omega, r, mu, S, p):
    q, k, v, alpha, omega, r = (_in(x) for x in (q, k, v, alpha, omega, r))
    N, H, dk = q.shape
    dv = v.shape[-1]
    S = np.array(S, dtype=np.float64, order="C", copy=True)
    p = np.array(p, dtype=np.float64, order="C", copy=True)
    o = np.zeros((N, H, dv))
    rc = getattr(_load(), name)(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                _ptr(omega), _ptr(r), float(mu), _ptr(S), _ptr(p), _ptr(o))
    if rc != 0:
        raise ValueError(f"{name}: bad arguments (rc={rc})")
    return {"o": o, "S": S, "p": p}


def step_diag(q, k, v, alpha, omega, r, mu, S, p):
    """One decode step.  q,k,alpha,omega [N,H,dk]; v [N,H,dv]; r [N,H];
    S [N,H,dk,dv]; p [N,H,dk].  Returns new (o, S, p); inputs untouched."""
    return _step("kdn_oracle_step_diag", q, k, v, alpha, omega, r, mu, S, p)


def step_iso(q, k, v, alpha, omega, r, mu, S, p):
    """Isotropic decode step: alpha, omega, r [N,H]; p [N,H]."""
    return _step("kdn_oracle_step_iso", q, k, v, alpha, omega, r, mu, S, p)


def step_isoc(q, k, v, alpha, omega, r, mu, S, p):
    """Per-channel-decay isotropic decode step: alpha [N,H,dk]; omega, r [N,H]; p [N,H]."""
    return _step("kdn_oracle_step_isoc", q, k, v, alpha, omega, r, mu, S, p)


_VARIANTS = {"diagonal": 0, "isotropic": 1, "isochannel": 2}


def _backward_grouped(q, k, v, alpha, omega, r, c0, mu, dO, dS_T, dp_T, S0, p0):
    """Adjoint of forward_grouped: the groups are independent diagonal
    recurrences on their value columns that share q, k, alpha, omega, so the
    gradients of the shared inputs are the sums over the groups of each
    group's diagonal adjoint, and those of v, r, S0, p0 are the groups' own."""
    r = np.asarray(r)
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    G = r.shape[-1]
    gw = dv // G
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
           "dalpha": np.zeros((B, T, H, dk)), "domega": np.zeros((B, T, H, dk)), "dr": np.zeros((B, T, H, G)),
           "dS0": np.zeros((B, H, dk, dv)), "dp0": np.zeros((B, H, G, dk)), "dc0": np.zeros(H)}
    for g in range(G):
        cols = slice(g * gw, (g + 1) * gw)
        res = backward(q, k, np.asarray(v)[..., cols], alpha, omega, r[..., g], c0, mu,
                       None if dO is None else np.asarray(dO)[..., cols],
                       None if dS_T is None else np.asarray(dS_T)[..., cols],
                       None if dp_T is None else np.asarray(dp_T)[:, :, g],
                       None if S0 is None else np.asarray(S0)[..., cols],
                       None if p0 is None else np.asarray(p0)[:, :, g], "diagonal")
        for n in ("dq", "dk", "dalpha", "domega", "dc0"):
            out[n] += res[n]
        out["dv"][..., cols] = res["dv"]
        out["dr"][..., g] = res["dr"]
        out["dS0"][..., cols] = res["dS0"]
        out["dp0"][:, :, g] = res["dp0"]
    return out


def backward(q, k, v, alpha, omega, r, c0, mu, dO=None, dS_T=None, dp_T=None, S0=None, p0=None,
             variant="diagonal"):
    """Gradients of L = sum(dO*o) + sum(dS_T*S_T) + sum(dp_T*p_T) for the
    forward of ``variant`` on these inputs (any of dO, dS_T, dp_T may be None
    for zero).  Returns dict dq, dk, dv, dalpha, domega, dr (input layouts),
    dS0 [B,H,dk,dv], dp0 [B,H,dk] (isotropic forms [B,H]; grouped noise
    [B,H,G,dk], dr [B,T,H,G]) and dc0 [H] (the sum of dp0 over batch, groups
    and channels: the c0 gradient when p0 is None)."""
    if variant == "grouped":
        return _backward_grouped(q, k, v, alpha, omega, r, c0, mu, dO, dS_T, dp_T, S0, p0)
    var = _VARIANTS[variant]
    q, k, v, alpha, omega, r = (_in(x) for x in (q, k, v, alpha, omega, r))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    c0 = _in(np.broadcast_to(np.asarray(c0, np.float64), (H,)))
    S0, p0, dO, dS_T, dp_T = (_f64(x) for x in (S0, p0, dO, dS_T, dp_T))
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dalpha": np.zeros_like(alpha), "domega": np.zeros_like(omega), "dr": np.zeros_like(r),
           "dS0": np.zeros((B, H, dk, dv)), "dp0": np.zeros((B, H, dk) if var == 0 else (B, H)),
           "dc0": np.zeros(H)}
    rc = _load().kdn_oracle_backward(
        var, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0),
        float(mu), _ptr(S0), _ptr(p0), _ptr(dO), _ptr(dS_T), _ptr(dp_T),
        *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0", "dc0")))
    if rc != 0:
        raise ValueError(f"backward: bad arguments (rc={rc})")
    return out


R_MIN = 0.01  # floor of the observation noise (summary page, method step 1)


def sigmoid(z):
    """Logistic function 1 / (1 + e^-z) in fp64, evaluated so that no
    exponential overflows: e^-|z| lies in (0, 1]."""
    z = np.asarray(z, np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(z):
    """log(1 + e^z) in fp64 as max(z, 0) + log1p(e^-|z|) (no overflow, no
    cancellation for large |z|)."""
    z = np.asarray(z, np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def gates(z_alpha, z_omega, z_r):
    """The gate step of the diagonal layer (summary page, method step 1):
    per-channel decay alpha = sigmoid(z_alpha), per-channel process noise
    omega = softplus(z_omega), per-token observation noise
    r = 0.01 + softplus(z_r).  The pre-activations are what the token's
    projections produce; the projections themselves are not part of this
    step.  Returns (alpha, omega, r) in fp64."""
    return sigmoid(_f64(z_alpha)), softplus(_f64(z_omega)), R_MIN + softplus(_f64(z_r))


NORM_EPS = 1e-6  # smallest norm l2norm divides by (a zero row stays zero)


def l2norm(x):
    """Each row of x (last axis: the d_k channels of one token-head) divided by
    its Euclidean norm, in fp64: the unit-norm keys the summary page's
    information scaling mu = d_k assumes (core method), queries alike.  Rows
    of norm below NORM_EPS are divided by NORM_EPS."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def prologue(q, k, z_alpha, z_omega, z_r):
    """The step before the recurrence (summary page, method step 1, and the
    unit-norm keys of the core method): q and k L2-normalised per
    token-head, then the gates.  Returns (q_hat, k_hat, alpha, omega, r)."""
    alpha, omega, r = gates(z_alpha, z_omega, z_r)
    return l2norm(q), l2norm(k), alpha, omega, r


def forward_gated(q, k, v, z_alpha, z_omega, z_r, c0, mu, S0=None, p0=None, variant="diagonal"):
    """The forward fed through ``prologue``: q and k normalised, the gates on
    the pre-activations, then ``forward_diag`` / ``forward_iso`` /
    ``forward_isoc`` (the gates are elementwise, so they apply to every
    variant's layouts alike)."""
    qh, kh, alpha, omega, r = prologue(q, k, z_alpha, z_omega, z_r)
    fn = {"diagonal": forward_diag, "isotropic": forward_iso, "isochannel": forward_isoc}[variant]
    return fn(qh, kh, v, alpha, omega, r, c0, mu, S0=S0, p0=p0)


def l2norm_backward(x, dxh):
    """Cotangent of the raw rows x given the cotangent dxh of l2norm(x): with
    n = |x| (>= NORM_EPS), dx = (dxh - xh (xh . dxh)) / n; below NORM_EPS the
    map is x / NORM_EPS and dx = dxh / NORM_EPS."""
    x, dxh = _f64(x), _f64(dxh)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    big = n >= NORM_EPS
    nn = np.where(big, n, NORM_EPS)
    xh = x / nn
    proj = np.sum(xh * dxh, axis=-1, keepdims=True)
    return np.where(big, (dxh - xh * proj) / nn, dxh / NORM_EPS)


def backward_gated(q, k, v, z_alpha, z_omega, z_r, c0, mu, dO=None, dS_T=None, dp_T=None, S0=None, p0=None,
                   variant="diagonal"):
    """Gradients of ``forward_gated``: ``backward`` on the prologue's values,
    then the chain rule through it: d q = l2norm_backward(q, d q_hat) (and k
    alike), d z_alpha = d alpha sigmoid'(z_alpha) with sigmoid' = sigmoid
    (1 - sigmoid), d z_omega = d omega sigmoid(z_omega) and d z_r = d r
    sigmoid(z_r) (softplus' = sigmoid).
    Returns dq, dk, dv, dz_alpha, dz_omega, dz_r, dS0, dp0, dc0."""
    qh, kh, alpha, omega, r = prologue(q, k, z_alpha, z_omega, z_r)
    g = backward(qh, kh, v, alpha, omega, r, c0, mu, dO=dO, dS_T=dS_T, dp_T=dp_T, S0=S0, p0=p0, variant=variant)
    out = {n: g[n] for n in ("dv", "dS0", "dp0", "dc0")}
    out["dq"] = l2norm_backward(q, g["dq"])
    out["dk"] = l2norm_backward(k, g["dk"])
    out["dz_alpha"] = g["dalpha"] * alpha * (1.0 - alpha)
    out["dz_omega"] = g["domega"] * sigmoid(_f64(z_omega))
    out["dz_r"] = g["dr"] * sigmoid(_f64(z_r))
    return out

