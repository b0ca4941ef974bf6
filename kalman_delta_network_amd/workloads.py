"""Seeded synthetic workloads for the KDN mixer recurrence.

This module only draws inputs.  It holds none of the recurrence's arithmetic,
so the GPU library, the fp64 oracle, the tests and the benchmark can all use
the same inputs without sharing any part of the computation.

Recipe (every tensor is drawn in float32 from ``numpy.random.default_rng``,
in the fixed order q, k, v, alpha, omega, r, c0; ``N(m, s)`` means mean m and
standard deviation s):

* q, k ~ N(0, 1), each (b, t, h) row L2-normalised over its d_k channels;
* v ~ N(0, 1);
* alpha = sigmoid(N(alpha_loc, 0.5)) per channel (isotropic: per head-token;
  isotropic with per-channel decay: per channel);
* omega = softplus(N(omega_loc, 1)) per channel (both isotropic forms: per
  head-token);
* r = 0.01 + softplus(N(0, 1)) per head-token (the pages' r_min = 0.01; the
  grouped variant: per head-token and group of value columns);
* c0 = 1.0 per head, or U(0.5, 2) per head;
* decode state: S0 ~ N(0, 0.1), p0 ~ U(0.1, 1) (isotropic: one p0 per head);
* packed variable-length batches: sequence lengths ~ U{lo, hi} (integers,
  both ends included), then the tokens of all sequences drawn as one
  [total, H] grid in the order above, then c0.

For bf16 workloads every tensor above except c0, S0 and p0 is then rounded
to bf16 (round to nearest, ties to even) and returned as float32 arrays that
hold exactly the bf16 values, so both sides of a comparison see identical
numbers.  The shapes are those of the 750M and 1.3B mixer layers of the
"Kalman Delta Networks" pages (d_k = d_v = 128, 16 heads).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str          # "diagonal", "isotropic" or "isochannel" (isotropic with per-channel decay)
    dtype: str            # "f32" or "bf16": dtype of q, k, v, alpha, omega, r and o
    B: int
    T: int
    H: int
    dk: int
    dv: int
    mu: float
    c0: str               # "one" or "uniform"
    seed: int
    alpha_loc: float = 2.0
    omega_loc: float = -4.0
    decode_steps: int = 0  # > 0: a decode workload with B sequences and T = 1 per step
    rgroups: int = 1       # "grouped" variant: observation noise r per group of d_v / rgroups value columns

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "diag_f32_b1_t256_h2_d64": Workload(
        "diag_f32_b1_t256_h2_d64", "diagonal", "f32", 1, 256, 2, 64, 64, 64.0, "one", 1000),
    "diag_bf16_b8_t4096_h16_d128": Workload(
        "diag_bf16_b8_t4096_h16_d128", "diagonal", "bf16", 8, 4096, 16, 128, 128, 128.0,
        "uniform", 1001),
    "iso_bf16_b8_t4096_h16_d128": Workload(
        "iso_bf16_b8_t4096_h16_d128", "isotropic", "bf16", 8, 4096, 16, 128, 128, 128.0,
        "uniform", 1002),
    "diag_bf16_b1_t65536_h16_d128": Workload(
        "diag_bf16_b1_t65536_h16_d128", "diagonal", "bf16", 1, 65536, 16, 128, 128, 128.0,
        "one", 1003, alpha_loc=4.0),
    "isoch_bf16_b8_t4096_h16_d128": Workload(
        "isoch_bf16_b8_t4096_h16_d128", "isochannel", "bf16", 8, 4096, 16, 128, 128, 128.0,
        "uniform", 1006),
    # grouped observation noise: one r per group of 64 value columns (2 groups)
    "grouped_bf16_b8_t4096_h16_d128": Workload(
        "grouped_bf16_b8_t4096_h16_d128", "grouped", "bf16", 8, 4096, 16, 128, 128, 128.0,
        "uniform", 1007, rgroups=2),
    "decode_diag_bf16_n256_h16_d128_s1024": Workload(
        "decode_diag_bf16_n256_h16_d128_s1024", "diagonal", "bf16", 256, 1, 16, 128, 128, 128.0,
        "one", 1004, decode_steps=1024),
    "decode_iso_bf16_n256_h16_d128_s1024": Workload(
        "decode_iso_bf16_n256_h16_d128_s1024", "isotropic", "bf16", 256, 1, 16, 128, 128, 128.0,
        "one", 1007, decode_steps=1024),
}
# the workloads in the order they are listed in the benchmark table
WORKLOAD_ORDER = list(WORKLOADS)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _softplus(x):
    return np.log1p(np.exp(x)).astype(np.float32)


def _l2norm(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _normal(rng, shape, loc=0.0, scale=1.0):
    z = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    if loc != 0.0:
        z += np.float32(loc)
    return z


def _draw_tokens(rng, w: Workload, lead: tuple) -> dict:
    """Draw q, k, v, alpha, omega, r with leading shape ``lead`` (e.g. (B,T,H))."""
    alpha_shape = lead + (w.dk,) if w.variant in ("diagonal", "isochannel", "grouped") else lead
    omega_shape = lead + (w.dk,) if w.variant in ("diagonal", "grouped") else lead
    r_shape = lead + (w.rgroups,) if w.variant == "grouped" else lead
    out = {
        "q": _l2norm(_normal(rng, lead + (w.dk,))),
        "k": _l2norm(_normal(rng, lead + (w.dk,))),
        "v": _normal(rng, lead + (w.dv,)),
        "alpha": _sigmoid(_normal(rng, alpha_shape, w.alpha_loc, 0.5)),
        "omega": _softplus(_normal(rng, omega_shape, w.omega_loc, 1.0)),
        "r": (np.float32(0.01) + _softplus(_normal(rng, r_shape))).astype(np.float32),
    }
    if w.dtype == "bf16":
        out = {key: round_bf16(val) for key, val in out.items()}
    return out


def _draw_c0(rng, w: Workload) -> np.ndarray:
    if w.c0 == "uniform":
        return rng.uniform(0.5, 2.0, size=w.H).astype(np.float32)
    return np.ones(w.H, dtype=np.float32)


def forward_inputs(w: Workload) -> dict:
    """All inputs of one forward call: q,k,v,alpha,omega,r (float32 arrays that
    hold the exact values of ``w.dtype``) and c0 [H] float32."""
    rng = np.random.default_rng(w.seed)
    out = _draw_tokens(rng, w, (w.B, w.T, w.H))
    out["c0"] = _draw_c0(rng, w)
    return out


def gated_inputs(w: Workload) -> dict:
    """Inputs of one gated forward, the step before the recurrence still to
    do: raw q, k ~ N(0, 1) (the gated forward normalises them), v as in
    ``forward_inputs`` and, in place of alpha, omega and r, their gate
    pre-activations z_alpha ~ N(alpha_loc, 0.5), z_omega ~ N(omega_loc, 1),
    z_r ~ N(0, 1) in the variant's layouts (the distributions whose gated
    values ``forward_inputs`` draws), all rounded to bf16 for bf16 workloads;
    c0 [H]."""
    rng = np.random.default_rng([w.seed, 0x6A])
    lead = (w.B, w.T, w.H)
    out = {
        "q": _normal(rng, lead + (w.dk,)),
        "k": _normal(rng, lead + (w.dk,)),
        "v": _normal(rng, lead + (w.dv,)),
        "z_alpha": _normal(rng, lead + (w.dk,) if w.variant in ("diagonal", "isochannel") else lead,
                           w.alpha_loc, 0.5),
        "z_omega": _normal(rng, lead + (w.dk,) if w.variant == "diagonal" else lead, w.omega_loc, 1.0),
        "z_r": _normal(rng, lead),
    }
    if w.dtype == "bf16":
        out = {key: round_bf16(val) for key, val in out.items()}
    out["c0"] = _draw_c0(rng, w)
    return out


# packed variable-length serving batch: 32 sequences of 256..1792 tokens
# (about 32k tokens in all, the token count of the main forward workload)
VARLEN = Workload("varlen_diag_bf16_n32_h16_d128", "diagonal", "bf16", 32, 0, 16, 128, 128, 128.0,
                  "uniform", 1005)
VARLEN_RANGE = (256, 1792)


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n sequence lengths drawn uniformly from lo..hi (inclusive), int64."""
    return np.random.default_rng([seed, 0x5E]).integers(lo, hi + 1, size=n)


def varlen_inputs(w: Workload, lengths) -> dict:
    """Inputs of one packed forward over len(lengths) sequences: q,k,v,alpha,
    omega,r with leading shape [total, H] (rows of sequence n are
    cu_seqlens[n] .. cu_seqlens[n+1]-1), cu_seqlens int32 [N+1], c0 [H]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    rng = np.random.default_rng(w.seed)
    out = _draw_tokens(rng, w, (int(cu[-1]), w.H))
    out["cu_seqlens"] = cu
    out["c0"] = _draw_c0(rng, w)
    return out


def decode_state(w: Workload) -> dict:
    """Initial carried state of a decode workload: S0 [N,H,dk,dv], p0 [N,H,dk]
    (isotropic: [N,H]) float32, N = w.B."""
    rng = np.random.default_rng([w.seed, 0xD0])
    S0 = _normal(rng, (w.B, w.H, w.dk, w.dv), 0.0, 0.1)
    pshape = {"diagonal": (w.B, w.H, w.dk), "grouped": (w.B, w.H, w.rgroups, w.dk)}.get(w.variant, (w.B, w.H))
    p0 = rng.uniform(0.1, 1.0, size=pshape).astype(np.float32)
    return {"S0": S0, "p0": p0}


def decode_tokens(w: Workload, step: int) -> dict:
    """The token of decode step ``step`` for all N = w.B sequences:
    q,k,alpha,omega [N,H,dk] (isotropic alpha, omega [N,H]), v [N,H,dv], r [N,H]."""
    rng = np.random.default_rng([w.seed, 0x70, step])
    return _draw_tokens(rng, w, (w.B, w.H))


def gated_decode_tokens(w: Workload, step: int) -> dict:
    """The token of decode step ``step`` for all N = w.B sequences, with gate
    pre-activations in the variant's layouts (q, k [N,H,dk], v [N,H,dv],
    z_r [N,H]; distributions as ``gated_inputs``)."""
    rng = np.random.default_rng([w.seed, 0x71, step])
    lead = (w.B, w.H)
    out = {
        "q": _l2norm(_normal(rng, lead + (w.dk,))),
        "k": _l2norm(_normal(rng, lead + (w.dk,))),
        "v": _normal(rng, lead + (w.dv,)),
        "z_alpha": _normal(rng, lead + (w.dk,) if w.variant in ("diagonal", "isochannel") else lead,
                           w.alpha_loc, 0.5),
        "z_omega": _normal(rng, lead + (w.dk,) if w.variant == "diagonal" else lead, w.omega_loc, 1.0),
        "z_r": _normal(rng, lead),
    }
    if w.dtype == "bf16":
        out = {key: round_bf16(val) for key, val in out.items()}
    return out


def backward_cotangents(w: Workload, with_state: bool = True) -> dict:
    """Cotangents of one backward call: dO ~ N(0, 1) [B,T,H,dv] (rounded to
    bf16 for bf16 workloads), and with ``with_state`` dS_T ~ N(0, 0.1)
    [B,H,dk,dv] and dp_T ~ N(0, 0.1) [B,H,dk] (isotropic forms [B,H]) in
    float32; without it those two are None."""
    rng = np.random.default_rng([w.seed, 0xBA])
    dO = _normal(rng, (w.B, w.T, w.H, w.dv))
    if w.dtype == "bf16":
        dO = round_bf16(dO)
    out = {"dO": dO, "dS_T": None, "dp_T": None}
    if with_state:
        out["dS_T"] = _normal(rng, (w.B, w.H, w.dk, w.dv), 0.0, 0.1)
        pshape = {"diagonal": (w.B, w.H, w.dk), "grouped": (w.B, w.H, w.rgroups, w.dk)}.get(w.variant, (w.B, w.H))
        out["dp_T"] = _normal(rng, pshape, 0.0, 0.1)
    return out
