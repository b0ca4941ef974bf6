"""MI355X (gfx950) implementation of the Kalman Delta Network mixer recurrence.

Thin Python binding of the C ABI in ``include/kdn.h`` (``libkdn.so``, built by
``kalman_delta_network_amd.build``).  This module only marshals arguments:
it checks tensor dtypes, shapes and devices, allocates outputs with PyTorch
and passes raw device pointers plus the current HIP stream to the library.
Every step of the recurrence runs in the library's kernels; there is no
fallback of any kind, and calling into a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkdn.so")

KDN_DIAGONAL, KDN_ISOTROPIC = 0, 1
KDN_F32, KDN_BF16 = 0, 1
(KDN_OK, KDN_ERR_NULL, KDN_ERR_SHAPE, KDN_ERR_UNSUPPORTED, KDN_ERR_VALUE, KDN_ERR_HIP, KDN_ERR_ALIAS,
 KDN_ERR_WORKSPACE) = range(8)
ALGOS = {"auto": 0, "recurrent": 1, "chunked": 2, "chunked_wide": 3, "chunked_narrow": 4}
KDN_ISOTROPIC_CHANNEL = 2
KDN_DIAGONAL_GROUPED = 3
VARIANTS = {"diagonal": KDN_DIAGONAL, "isotropic": KDN_ISOTROPIC, "isochannel": KDN_ISOTROPIC_CHANNEL,
            "grouped": KDN_DIAGONAL_GROUPED}
GROUP_COLS = 64  # value columns per observation-noise group of the grouped variant


def _gate_shapes(var, lead, dk):
    """(alpha shape, omega shape) of a variant for token dims ``lead``."""
    alpha = lead + (dk,) if var != KDN_ISOTROPIC else lead
    omega = lead + (dk,) if var in (KDN_DIAGONAL, KDN_DIAGONAL_GROUPED) else lead
    return alpha, omega


def _r_shape(var, lead, dv):
    """Shape of r: one entry per head-token, or per group of value columns."""
    return lead + (dv // GROUP_COLS,) if var == KDN_DIAGONAL_GROUPED else lead


def _p_shape(var, lead, dk, dv):
    """Shape of the uncertainty state for state dims ``lead`` (e.g. (B, H))."""
    if var == KDN_DIAGONAL:
        return lead + (dk,)
    if var == KDN_DIAGONAL_GROUPED:
        return lead + (dv // GROUP_COLS, dk)
    return lead

# exported symbols of include/kdn.h
SYMBOLS = ("kdn_forward", "kdn_forward_algo", "kdn_forward_varlen", "kdn_forward_gated",
           "kdn_forward_varlen_gated", "kdn_step", "kdn_step_gated", "kdn_backward_gated",
           "kdn_backward_gated_workspace_size", "kdn_backward_gated_workspace_size_for", "kdn_backward_noalloc",
           "kdn_forward_split",
           "kdn_forward_split_segments", "kdn_forward_split_workspace_size", "kdn_validate_forward_split",
           "kdn_validate_forward", "kdn_validate_forward_varlen", "kdn_validate_forward_gated",
           "kdn_validate_step", "kdn_backward", "kdn_backward_workspace_size", "kdn_backward_workspace_size_for",
           "kdn_validate_backward", "kdn_status_string", "kdn_last_error", "kdn_version")

_lib = None


class KDNError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libkdn.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m kalman_delta_network_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fwd = [P, P, P, P, P, P, P, F, I, I, I, I, I, I, I, P, P, P, P, P]
    lib.kdn_forward.argtypes = fwd + [P]
    lib.kdn_forward_algo.argtypes = fwd + [P, I]
    lib.kdn_validate_forward.argtypes = fwd + [I]
    lib.kdn_forward_gated.argtypes = fwd + [P, I]
    lib.kdn_forward_split.argtypes = fwd + [I, P, ctypes.c_size_t, P]
    lib.kdn_validate_forward_split.argtypes = fwd + [I, P, ctypes.c_size_t]
    lib.kdn_forward_split_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kdn_forward_split_workspace_size.restype = ctypes.c_size_t
    lib.kdn_forward_split_segments.argtypes = [I, I, I, I, I, I]
    lib.kdn_forward_split_segments.restype = I
    lib.kdn_validate_forward_gated.argtypes = fwd + [I]
    step = [P, P, P, P, P, P, F, I, I, I, I, I, I, P, P, P]
    lib.kdn_step.argtypes = step + [P]
    lib.kdn_validate_step.argtypes = step
    varlen = [P, P, P, P, P, P, P, P, P, F, I, I, I, I, I, I, I, P, P, P, P, P]
    lib.kdn_forward_varlen.argtypes = varlen + [P, I]
    lib.kdn_forward_varlen_gated.argtypes = varlen + [P, I]
    lib.kdn_step_gated.argtypes = step + [P]
    lib.kdn_validate_forward_varlen.argtypes = varlen + [I]
    bwd = fwd[:17] + [P] * 12
    lib.kdn_backward.argtypes = bwd + [P, ctypes.c_size_t, P]
    lib.kdn_validate_backward.argtypes = bwd + [P, ctypes.c_size_t]
    lib.kdn_backward_workspace_size.argtypes = [I, I, I, I, I]
    lib.kdn_backward_workspace_size.restype = ctypes.c_size_t
    lib.kdn_backward_workspace_size_for.argtypes = [I, I, I, I, I, I, I]
    lib.kdn_backward_workspace_size_for.restype = ctypes.c_size_t
    lib.kdn_backward_gated.argtypes = bwd + [P, ctypes.c_size_t, P]
    lib.kdn_backward_noalloc.argtypes = bwd + [P]
    lib.kdn_backward_gated_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.kdn_backward_gated_workspace_size.restype = ctypes.c_size_t
    lib.kdn_backward_gated_workspace_size_for.argtypes = [I, I, I, I, I, I, I]
    lib.kdn_backward_gated_workspace_size_for.restype = ctypes.c_size_t
    for fn in (lib.kdn_forward, lib.kdn_forward_algo, lib.kdn_validate_forward, lib.kdn_step,
               lib.kdn_validate_step, lib.kdn_forward_varlen, lib.kdn_validate_forward_varlen,
               lib.kdn_backward, lib.kdn_validate_backward, lib.kdn_version, lib.kdn_forward_gated,
               lib.kdn_validate_forward_gated, lib.kdn_forward_varlen_gated, lib.kdn_step_gated,
               lib.kdn_backward_gated, lib.kdn_backward_noalloc):
        fn.restype = I
    lib.kdn_status_string.argtypes = [I]
    lib.kdn_status_string.restype = ctypes.c_char_p
    lib.kdn_last_error.argtypes = []
    lib.kdn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != KDN_OK:
        lib = load_library()
        detail = (lib.kdn_last_error() or lib.kdn_status_string(status)).decode()
        raise KDNError(status, where, detail)


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDN_BF16
    if t.dtype == torch.float32:
        return KDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def forward(q, k, v, alpha, omega, r, c0, mu, variant="diagonal", S0=None, p0=None,
            algo="auto", out=None):
    """KDN forward over [B,T,H,*] tensors on one GPU.

    q, k [B,T,H,dk]; v [B,T,H,dv]; alpha, omega [B,T,H,dk] (isotropic [B,T,H];
    "isochannel", the isotropic form with per-channel decay: alpha [B,T,H,dk],
    omega [B,T,H]); r [B,T,H] ("grouped", grouped observation noise: [B,T,H,dv/64])
    -- all float32 or all bfloat16.  c0 [H] float32 (may be None if p0 is given);
    S0 [B,H,dk,dv] / p0 [B,H,dk] (isotropic [B,H]; grouped [B,H,dv/64,dk])
    float32 or None.
    Returns (o, S_T, p_T); ``out`` may supply preallocated (o, S_T, p_T).
    """
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    ashape, wshape = _gate_shapes(var, (B, T, H), dk)
    pshape = _p_shape(var, (B, H), dk, dv)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("alpha", alpha, ashape), ("omega", omega, wshape), ("r", r, _r_shape(var, (B, T, H), dv))):
        _need(t, name, shp, dt, dev)
    if c0 is not None:
        _need(c0, "c0", (H,), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if p0 is not None:
        _need(p0, "p0", pshape, torch.float32, dev)
    if out is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        p_T = torch.empty(pshape, dtype=torch.float32, device=dev)
    else:
        o, S_T, p_T = out
        _need(o, "o", (B, T, H, dv), dt, dev)
        _need(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
        _need(p_T, "p_T", pshape, torch.float32, dev)
    st = lib.kdn_forward_algo(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0),
                              float(mu), var, _dtype_code(q), B, T, H, dk, dv, _ptr(S0), _ptr(p0),
                              _ptr(o), _ptr(S_T), _ptr(p_T), _stream(dev), ALGOS[algo])
    _check(st, "kdn_forward")
    return o, S_T, p_T


def forward_split_segments(B, T, H, dk, dv, segments=0) -> int:
    """Segments ``forward_split`` cuts each sequence into on this device."""
    return int(load_library().kdn_forward_split_segments(B, T, H, dk, dv, segments))


def forward_split_workspace_size(B, T, H, dk, dv, segments=0) -> int:
    """Workspace bytes of ``forward_split`` (0: no split for these sizes)."""
    return int(load_library().kdn_forward_split_workspace_size(B, T, H, dk, dv, segments))


def forward_split(q, k, v, alpha, omega, r, c0, mu, S0=None, p0=None, segments=0, workspace=None, out=None):
    """Diagonal KDN forward (bf16) with each sequence cut into segments that
    run concurrently, for batches too small to fill the device.  segments: 0
    chooses from the device, > 0 asks for about that many.  ``workspace``: a
    uint8 device tensor of at least forward_split_workspace_size(...) bytes,
    allocated here when None.  Arguments and results as ``forward``."""
    torch = _torch()
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("alpha", alpha, (B, T, H, dk)), ("omega", omega, (B, T, H, dk)), ("r", r, (B, T, H))):
        _need(t, name, shp, dt, dev)
    if c0 is not None:
        _need(c0, "c0", (H,), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if p0 is not None:
        _need(p0, "p0", (B, H, dk), torch.float32, dev)
    if out is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        p_T = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    else:
        o, S_T, p_T = out
    need = int(lib.kdn_forward_split_workspace_size(B, T, H, dk, dv, segments))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.kdn_forward_split(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0), float(mu),
                               VARIANTS["diagonal"], _dtype_code(q), B, T, H, dk, dv, _ptr(S0), _ptr(p0), _ptr(o),
                               _ptr(S_T), _ptr(p_T), int(segments), _ptr(workspace), int(workspace.numel()),
                               _stream(dev))
    _check(st, "kdn_forward_split")
    return o, S_T, p_T


def forward_gated(q, k, v, z_alpha, z_omega, z_r, c0, mu, variant="diagonal", S0=None, p0=None, algo="auto",
                  out=None):
    """KDN forward with the step before the recurrence inside the kernel: q
    and k are raw (each [dk] row is divided by max(|row|, 1e-6)); z_alpha,
    z_omega and z_r are pre-activations in the layouts ``forward`` gives
    alpha, omega and r for the variant ("diagonal", "isotropic" or
    "isochannel"), and the kernel uses alpha = sigmoid(z_alpha),
    omega = softplus(z_omega), r = 0.01 + softplus(z_r).  Other arguments and
    results as ``forward``."""
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    ashape, wshape = _gate_shapes(var, (B, T, H), dk)
    pshape = _p_shape(var, (B, H), dk, dv)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("z_alpha", z_alpha, ashape), ("z_omega", z_omega, wshape), ("z_r", z_r, (B, T, H))):
        _need(t, name, shp, dt, dev)
    if c0 is not None:
        _need(c0, "c0", (H,), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if p0 is not None:
        _need(p0, "p0", pshape, torch.float32, dev)
    if out is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        p_T = torch.empty(pshape, dtype=torch.float32, device=dev)
    else:
        o, S_T, p_T = out
        _need(o, "o", (B, T, H, dv), dt, dev)
        _need(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
        _need(p_T, "p_T", pshape, torch.float32, dev)
    st = lib.kdn_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z_alpha), _ptr(z_omega), _ptr(z_r), _ptr(c0),
                               float(mu), var, _dtype_code(q), B, T, H, dk, dv, _ptr(S0), _ptr(p0),
                               _ptr(o), _ptr(S_T), _ptr(p_T), _stream(dev), ALGOS[algo])
    _check(st, "kdn_forward_gated")
    return o, S_T, p_T


def longest_first(cu_seqlens):
    """Scheduling order for forward_varlen from host-side offsets (a list,
    numpy array or CPU tensor of N+1 ints): sequence indices by decreasing
    length, ties in index order, as an int32 numpy array."""
    import numpy as np
    cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
    return np.argsort(-(cu[1:] - cu[:-1]), kind="stable").astype(np.int32)


def forward_varlen(q, k, v, alpha, omega, r, c0, cu_seqlens, mu, variant="diagonal", S0=None, p0=None,
                   algo="auto", out=None, order=None):
    """KDN forward over N sequences packed along the token axis.

    q, k [total,H,dk]; v [total,H,dv]; alpha, omega [total,H,dk] (isotropic
    [total,H]); r [total,H] -- float32 or bfloat16.  cu_seqlens: int32 device
    tensor [N+1] of token offsets (sequence n owns rows cu[n] .. cu[n+1]-1).
    c0 [H]; S0 [N,H,dk,dv] / p0 [N,H,dk] (isotropic [N,H]) float32 or None.
    order: int32 device tensor [N], the scheduling order (a permutation;
    ``longest_first`` of the host offsets balances the GPU), or None.
    Returns (o [total,H,dv], S_T [N,H,dk,dv], p_T); ``out`` may supply them.
    """
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    total, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens: expected a 1-D tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    ashape, wshape = _gate_shapes(var, (total, H), dk)
    pshape = _p_shape(var, (N, H), dk, dv)
    for name, t, shp in (("q", q, (total, H, dk)), ("k", k, (total, H, dk)), ("v", v, (total, H, dv)),
                         ("alpha", alpha, ashape), ("omega", omega, wshape), ("r", r, _r_shape(var, (total, H), dv))):
        _need(t, name, shp, dt, dev)
    if order is not None:
        _need(order, "order", (N,), torch.int32, dev)
    if c0 is not None:
        _need(c0, "c0", (H,), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if p0 is not None:
        _need(p0, "p0", pshape, torch.float32, dev)
    if out is None:
        o = torch.empty((total, H, dv), dtype=dt, device=dev)
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        p_T = torch.empty(pshape, dtype=torch.float32, device=dev)
    else:
        o, S_T, p_T = out
        _need(o, "o", (total, H, dv), dt, dev)
        _need(S_T, "S_T", (N, H, dk, dv), torch.float32, dev)
        _need(p_T, "p_T", pshape, torch.float32, dev)
    st = lib.kdn_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r),
                                _ptr(cu_seqlens), _ptr(order), _ptr(c0), float(mu), var, _dtype_code(q), N, total, H,
                                dk, dv, _ptr(S0), _ptr(p0), _ptr(o), _ptr(S_T), _ptr(p_T), _stream(dev),
                                ALGOS[algo])
    _check(st, "kdn_forward_varlen")
    return o, S_T, p_T


def step(q, k, v, alpha, omega, r, mu, S, p, variant="diagonal", o=None):
    """One decode step for N sequences; S [N,H,dk,dv] and p [N,H,dk]
    (isotropic [N,H]) float32 are updated in place.  Returns o [N,H,dv]."""
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    ashape, wshape = _gate_shapes(var, (N, H), dk)
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("v", v, (N, H, dv)),
                         ("alpha", alpha, ashape), ("omega", omega, wshape), ("r", r, _r_shape(var, (N, H), dv))):
        _need(t, name, shp, dt, dev)
    _need(S, "S", (N, H, dk, dv), torch.float32, dev)
    _need(p, "p", _p_shape(var, (N, H), dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _need(o, "o", (N, H, dv), dt, dev)
    st = lib.kdn_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), float(mu), var,
                      _dtype_code(q), N, H, dk, dv, _ptr(S), _ptr(p), _ptr(o), _stream(dev))
    _check(st, "kdn_step")
    return o


def step_gated(q, k, v, z_alpha, z_omega, z_r, mu, S, p, variant="diagonal", o=None):
    """One decode step from raw q, k (normalised per row inside the kernel)
    and gate pre-activations z_alpha, z_omega, z_r in the layouts ``step``
    gives alpha, omega, r (the kernel applies sigmoid, softplus and
    0.01 + softplus); S and p float32 are updated in place.
    Returns o [N,H,dv]."""
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    ashape, wshape = _gate_shapes(var, (N, H), dk)
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("v", v, (N, H, dv)),
                         ("z_alpha", z_alpha, ashape), ("z_omega", z_omega, wshape), ("z_r", z_r, (N, H))):
        _need(t, name, shp, dt, dev)
    _need(S, "S", (N, H, dk, dv), torch.float32, dev)
    _need(p, "p", _p_shape(var, (N, H), dk, dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _need(o, "o", (N, H, dv), dt, dev)
    st = lib.kdn_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z_alpha), _ptr(z_omega), _ptr(z_r), float(mu),
                            var, _dtype_code(q), N, H, dk, dv, _ptr(S), _ptr(p), _ptr(o), _stream(dev))
    _check(st, "kdn_step_gated")
    return o


def forward_varlen_gated(q, k, v, z_alpha, z_omega, z_r, c0, cu_seqlens, mu, variant="diagonal", S0=None,
                         p0=None, algo="auto", order=None):
    """``forward_varlen`` from raw q, k (normalised per row inside the
    kernel) and gate pre-activations z_alpha, z_omega, z_r in the layouts
    ``forward_varlen`` gives alpha, omega, r."""
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    total, H, dk = q.shape
    dv = v.shape[-1]
    N = int(cu_seqlens.shape[0]) - 1
    dev, dt = q.device, q.dtype
    ashape, wshape = _gate_shapes(var, (total, H), dk)
    pshape = _p_shape(var, (N, H), dk, dv)
    for name, t, shp in (("q", q, (total, H, dk)), ("k", k, (total, H, dk)), ("v", v, (total, H, dv)),
                         ("z_alpha", z_alpha, ashape), ("z_omega", z_omega, wshape), ("z_r", z_r, (total, H))):
        _need(t, name, shp, dt, dev)
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if order is not None:
        _need(order, "order", (N,), torch.int32, dev)
    if c0 is not None:
        _need(c0, "c0", (H,), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if p0 is not None:
        _need(p0, "p0", pshape, torch.float32, dev)
    o = torch.empty((total, H, dv), dtype=dt, device=dev)
    S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    p_T = torch.empty(pshape, dtype=torch.float32, device=dev)
    st = lib.kdn_forward_varlen_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z_alpha), _ptr(z_omega), _ptr(z_r),
                                      _ptr(cu_seqlens), _ptr(order), _ptr(c0), float(mu), var,
                                      _dtype_code(q), N, total, H, dk, dv, _ptr(S0), _ptr(p0), _ptr(o),
                                      _ptr(S_T), _ptr(p_T), _stream(dev), ALGOS[algo])
    _check(st, "kdn_forward_varlen_gated")
    return o, S_T, p_T


def backward_workspace_size(B, T, H, dk, dv, variant=None, dtype=None) -> int:
    """Bytes of device workspace for kdn_backward at these sizes: with
    ``variant`` and ``dtype`` (a torch dtype), the smallest it accepts for
    them (kdn_backward_workspace_size_for); without, the size that serves
    every variant and dtype with all pairs at once."""
    lib = load_library()
    if variant is None:
        return int(lib.kdn_backward_workspace_size(B, T, H, dk, dv))
    torch = _torch()
    code = {torch.bfloat16: KDN_BF16, torch.float32: KDN_F32}[dtype]
    return int(lib.kdn_backward_workspace_size_for(VARIANTS[variant], code, B, T, H, dk, dv))


def backward(q, k, v, alpha, omega, r, c0, mu, dO=None, dS_T=None, dp_T=None, variant="diagonal",
             S0=None, p0=None, workspace=None):
    """Gradients of L = sum(dO*o) + sum(dS_T*S_T) + sum(dp_T*p_T), where
    (o, S_T, p_T) = forward(q, k, v, alpha, omega, r, c0, mu, variant, S0, p0).

    Inputs as ``forward``; dO [B,T,H,dv] in the input dtype, dS_T
    [B,H,dk,dv] and dp_T [B,H,dk] (isotropic forms [B,H]) float32; any of the
    three may be None (zero).  ``workspace``: a uint8 device tensor of at
    least backward_workspace_size(..., variant, q.dtype) bytes, or None to
    allocate that many.
    Returns a dict of float32 tensors dq, dk, dv, dalpha, domega, dr (input
    layouts), dS0, dp0 and dc0 [H] (sum of dp0 over batch and channels).
    """
    return _backward(q, k, v, alpha, omega, r, c0, mu, dO, dS_T, dp_T, variant, S0, p0, workspace, False)


def backward_noalloc(q, k, v, alpha, omega, r, c0, mu, dO=None, dS_T=None, dp_T=None, variant="diagonal",
                     S0=None, p0=None, out=None):
    """``backward`` through kdn_backward_noalloc: the library's static device
    scratch replaces the workspace, so the C call allocates nothing (sizes
    whose workspace exceeds NOALLOC_SCRATCH_BYTES raise KDNError with
    KDN_ERR_WORKSPACE).  ``out``: an optional dict of preallocated gradient
    tensors (the keys ``backward`` returns); missing ones are allocated here,
    by torch, before the call."""
    return _backward(q, k, v, alpha, omega, r, c0, mu, dO, dS_T, dp_T, variant, S0, p0, None, False, noalloc=True,
                     out=out)


NOALLOC_SCRATCH_BYTES = 256 << 20  # KDN_NOALLOC_SCRATCH_BYTES of kdn.h


def backward_gated_workspace_size(B, T, H, dk, dv, variant="diagonal", dtype=None) -> int:
    """Bytes of device workspace for kdn_backward_gated at these sizes: with
    ``dtype`` (a torch dtype), the smallest it accepts for the variant and
    dtype; without, the size that serves every dtype with all pairs at once."""
    lib = load_library()
    if dtype is None:
        return int(lib.kdn_backward_gated_workspace_size(VARIANTS[variant], B, T, H, dk, dv))
    torch = _torch()
    code = {torch.bfloat16: KDN_BF16, torch.float32: KDN_F32}[dtype]
    return int(lib.kdn_backward_gated_workspace_size_for(VARIANTS[variant], code, B, T, H, dk, dv))


def backward_gated(q, k, v, z_alpha, z_omega, z_r, c0, mu, dO=None, dS_T=None, dp_T=None, variant="diagonal",
                   S0=None, p0=None, workspace=None):
    """Gradients of the gated forward (``forward_gated``) with respect to its
    inputs: the raw q, k and the gate pre-activations included.  Arguments as ``backward``
    with z_alpha, z_omega, z_r in place of alpha, omega, r; the workspace is
    backward_gated_workspace_size() bytes.  Returns dq, dk, dv, dz_alpha,
    dz_omega, dz_r, dS0, dp0, dc0."""
    g = _backward(q, k, v, z_alpha, z_omega, z_r, c0, mu, dO, dS_T, dp_T, variant, S0, p0, workspace, True)
    return {("dz_" + n[1:] if n in ("dalpha", "domega", "dr") else n): t for n, t in g.items()}


def _backward(q, k, v, alpha, omega, r, c0, mu, dO, dS_T, dp_T, variant, S0, p0, workspace, gated, noalloc=False,
              out=None):
    torch = _torch()
    lib = load_library()
    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    ashape, wshape = _gate_shapes(var, (B, T, H), dk)
    pshape = _p_shape(var, (B, H), dk, dv)
    rshape = _r_shape(var, (B, T, H), dv)
    names = ("z_alpha", "z_omega", "z_r") if gated else ("alpha", "omega", "r")
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         (names[0], alpha, ashape), (names[1], omega, wshape), (names[2], r, rshape)):
        _need(t, name, shp, dt, dev)
    if dO is not None:
        _need(dO, "dO", (B, T, H, dv), dt, dev)
    for name, t, shp in (("c0", c0, (H,)), ("S0", S0, (B, H, dk, dv)), ("p0", p0, pshape),
                         ("dS_T", dS_T, (B, H, dk, dv)), ("dp_T", dp_T, pshape)):
        if t is not None:
            _need(t, name, shp, torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dq": (B, T, H, dk), "dk": (B, T, H, dk), "dv": (B, T, H, dv), "dalpha": ashape, "domega": wshape,
              "dr": rshape, "dS0": (B, H, dk, dv), "dp0": pshape, "dc0": (H,)}
    out = out or {}
    g = {}
    for n, shp in shapes.items():
        if n in out:
            _need(out[n], n, shp, torch.float32, dev)
            g[n] = out[n]
        else:
            g[n] = torch.empty(shp, **f32)
    if noalloc:
        st = lib.kdn_backward_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0), float(mu), var, _dtype_code(q),
            B, T, H, dk, dv, _ptr(S0), _ptr(p0), _ptr(dO), _ptr(dS_T), _ptr(dp_T),
            *(_ptr(g[n]) for n in ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0", "dc0")), _stream(dev))
        _check(st, "kdn_backward_noalloc")
        return g
    need = (backward_gated_workspace_size(B, T, H, dk, dv, variant, dt) if gated
            else backward_workspace_size(B, T, H, dk, dv, variant, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    fn = lib.kdn_backward_gated if gated else lib.kdn_backward
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(omega), _ptr(r), _ptr(c0), float(mu),
            var, _dtype_code(q), B, T, H, dk, dv, _ptr(S0), _ptr(p0), _ptr(dO), _ptr(dS_T),
            _ptr(dp_T), *(_ptr(g[n]) for n in ("dq", "dk", "dv", "dalpha", "domega", "dr", "dS0", "dp0", "dc0")),
            _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "kdn_backward_gated" if gated else "kdn_backward")
    return g
