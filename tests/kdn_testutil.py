"""Shared helpers of the GPU parity tests (inputs to the device, error metric,
oracle on a sample of heads)."""
from __future__ import annotations

import numpy as np

import oracle
from kalman_delta_network_amd import workloads as wl

TOKEN_INPUTS = ("q", "k", "v", "alpha", "omega", "r")


def tol(dtype: str) -> float:
    """Max relative error allowed against the fp64 oracle: 1e-4 for fp32
    inputs, 2e-2 for bf16 inputs with fp32 state."""
    return 1e-4 if dtype == "f32" else 2e-2


def rel_err(x, ref) -> float:
    """max |x - ref| / max |ref| over one output tensor."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (scale if scale > 0 else 1.0))


def p_rel_err(x, ref) -> float:
    """Elementwise relative error of the uncertainty p, which is strictly
    positive: max |x - ref| / ref.  Unlike the per-tensor metric it does not
    hide errors on small channels."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(ref > 0), "the oracle's p must be positive"
    return float(np.max(np.abs(x - ref) / ref))


def check_forward(name, got, ref, dtype):
    """Compare (o, S_T, p_T) with the oracle's: the per-tensor metric on each
    and the elementwise one on p, every entry finite, all within tol(dtype).
    Returns the errors."""
    errs = {k: rel_err(g, ref[k]) for k, g in zip(("o", "S", "p"), got)}
    errs["p_elem"] = p_rel_err(got[2], ref["p"])
    print(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, g in zip(("o", "S", "p"), got):
        assert np.all(np.isfinite(np.asarray(g, np.float64))), (name, k, "non-finite")
    for k, e in errs.items():
        assert e <= tol(dtype), (name, k, e)
    return errs


def to_dev(x: dict, dtype: str, device):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(tdt).to(device) for n in TOKEN_INPUTS if n in x}
    if "c0" in x:
        out["c0"] = torch.from_numpy(np.ascontiguousarray(x["c0"], np.float32)).to(device)
    return out


def oracle_forward(w: wl.Workload, x: dict, S0=None, p0=None, trace=False):
    fn = {"diagonal": oracle.forward_diag, "isotropic": oracle.forward_iso,
          "isochannel": oracle.forward_isoc}[w.variant]
    return fn(**{n: x[n] for n in TOKEN_INPUTS}, c0=x["c0"], mu=w.mu, S0=S0, p0=p0, trace=trace)


def oracle_forward_heads(w: wl.Workload, x: dict, pairs):
    """Oracle on selected (b, h) pairs only; returns {(b,h): result}."""
    res = {}
    for b, h in pairs:
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1]) for n in TOKEN_INPUTS}
        sub["c0"] = x["c0"][h:h + 1]
        res[(b, h)] = oracle_forward(w, sub)
    return res


def sample_pairs(B: int, H: int, n: int, seed: int = 0):
    rng = np.random.default_rng(seed)
    allp = [(b, h) for b in range(B) for h in range(H)]
    idx = rng.choice(len(allp), size=min(n, len(allp)), replace=False)
    picked = {allp[i] for i in idx} | {(0, 0), (B - 1, H - 1)}
    return sorted(picked)


def check_dc0(dc0, dp0):
    """dc0 is the sum of dp0 over the batch and every axis after the head
    axis (the c0 gradient when p0 is not given): compare the kernel's dc0 with
    the kernel's own dp0 summed in fp64, relative to the sum of magnitudes (a
    sum's rounding and inherited errors scale with sum |terms|, not with
    |sum|).  dp0 itself is compared with the oracle elsewhere."""
    dp0 = np.asarray(dp0, np.float64)
    axes = (0,) + tuple(range(2, dp0.ndim))
    want = dp0.sum(axis=axes)
    scale = np.abs(dp0).sum(axis=axes)
    err = np.abs(np.asarray(dc0, np.float64) - want)
    assert np.all(err <= 1e-5 * np.maximum(scale, 1e-30)), (err, scale)


# Workspace sizes of the backward, restated from include/kdn.h

def r256(n):
    return (n + 255) // 256 * 256


def token_pair_bytes(T, dk, dv):
    # one (batch, head) pair on the token path, per 64-column tile: ceil(T/32) checkpoints of S
    # and of p (one copy per 8 value columns), a 32-token stash, and per token the tile's four
    # row sums and p_{t-1}
    nseg, nt = -(-T // 32), dv // 64
    return nt * (nseg * (64 * dk + 8 * dk) + 32 * 64 * dk + 5 * T * dk) * 4


def chunk_min_bytes(B, T, H, dk, dv):
    # the chunked backward's regions (include/kdn.h, kdn_backward_workspace_size_for): flags,
    # bf16 chunk-start states, chunk-start p, 8 per-token sums, the uncertainty segments' maps
    # (64 tokens each) of one slab, dp and dS carried between slabs, one slab's tile sums and
    # p_{t-1}; the slab is about 64k token-heads, a multiple of 512, at most the sequence
    U, nt, nch = B * H, dv // 64, -(-T // 32)
    per = -(-65536 // U)  # token-heads per pair, rounded up
    slab = min(nch * 32, max(512, -(-per // 512) * 512))
    regions = (U * 4, U * nt * nch * dk * 64 * 2, U * nch * dk * 4, U * T * 32, U * -(-slab // 64) * dk * 8,
               2 * U * dk * 4, U * dk * dv * 4, U * slab * nt * 4 * dk * 4, U * slab * dk * 4)
    return max(sum(r256(x) for x in regions), r256(U * 4) + token_pair_bytes(T, dk, dv))
