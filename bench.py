"""Benchmark of the KDN forward recurrence on one MI355X.

One step = one kdn_forward call over the diagonal bf16 mixer-layer workload
(B=8, T=4096, H=16, d_k=d_v=128, fp32 state), inputs resident in HBM.
Prints ONE JSON line with the throughput in tokens/s (B*T per call), the
HBM roofline of the forward kernel measured with HIP events on the stream it
runs on, and the fp64 CPU oracle's rate on the same workload.  Warm-up runs
at least W steps and at least 0.3 s of GPU work (the clock ramps up over the
first tens of milliseconds of sustained load).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--algo auto|recurrent|chunked]
                    [--no-cpu-baseline] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
CHUNK = 32  # tokens per chunk of the chunked forward
MAIN = "diag_bf16_b8_t4096_h16_d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _gate_elems(w) -> int:
    """alpha plus omega elements per token-head, and the r entries beyond one."""
    return {"diagonal": 2 * w.dk, "isotropic": 2, "isochannel": w.dk + 1,
            "grouped": 2 * w.dk + w.rgroups - 1}[w.variant]


def _pdim(w) -> int:
    """Entries of the uncertainty state per (batch, head)."""
    return {"diagonal": w.dk, "grouped": w.rgroups * w.dk}.get(w.variant, 1)


def forward_bytes(w) -> int:
    """Algorithmic HBM bytes of one forward call: every input read once, o
    written once in the input dtype, final state written, c0 read."""
    es = 2 if w.dtype == "bf16" else 4
    toks = w.B * w.T * w.H
    per_tok = es * (2 * w.dk + w.dv + _gate_elems(w) + 1) + es * w.dv
    pdim = _pdim(w)
    return toks * per_tok + w.B * w.H * (w.dk * w.dv + pdim) * 4 + w.H * 4


def varlen_bytes(w, total: int) -> int:
    """Algorithmic HBM bytes of one packed forward over w.B sequences holding
    `total` tokens in all: as forward_bytes, plus the N+1 offsets."""
    es = 2 if w.dtype == "bf16" else 4
    per_tok = es * (2 * w.dk + w.dv + _gate_elems(w) + 1) + es * w.dv
    pdim = _pdim(w)
    return total * w.H * per_tok + w.B * w.H * (w.dk * w.dv + pdim) * 4 + w.H * 4 + (w.B + 1) * 4


def step_bytes(w) -> int:
    """Algorithmic HBM bytes of one decode step: state read and written once,
    one token of inputs read, o written."""
    es = 2 if w.dtype == "bf16" else 4
    units = w.B * w.H
    pdim = _pdim(w)
    return units * (2 * 4 * (w.dk * w.dv + pdim) + es * (2 * w.dk + w.dv + _gate_elems(w) + 1) + es * w.dv)


def forward_flops(w) -> int:
    """Algorithmic matrix flops of one chunked forward: per token-head
    2 L (d_k + d_v) for the chunk's triangular L x L products (tril(Kt Kh^T),
    tril(Qt Kh^T), the solve and tril(Qt Kh^T) Dn) plus 6 d_k d_v for
    Kt S, Qt S and the state update, at L = CHUNK."""
    return w.B * w.T * w.H * (2 * CHUNK * (w.dk + w.dv) + 6 * w.dk * w.dv)


def backward_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: the forward's inputs and
    dO read once, the fp32 gradients of q, k, v, alpha, omega, r written
    once, plus dS0, dp0 and dc0 (the recomputation checkpoints are the
    implementation's own traffic and are not counted)."""
    es = 2 if w.dtype == "bf16" else 4
    toks = w.B * w.T * w.H
    n_in = 2 * w.dk + w.dv + _gate_elems(w) + 1
    pdim = _pdim(w)
    return toks * (es * (n_in + w.dv) + 4 * n_in) + w.B * w.H * (w.dk * w.dv + pdim) * 4 + 2 * w.H * 4


def chunked_workgroups(w, cus: int = 256) -> int:
    """Workgroups of the chunked forward under the library's own choice: one
    per (batch, head) and 64 value columns, or per 32 columns when the
    64-column tiling fills at most half of the device's compute units."""
    wide = w.B * w.H * (w.dv // 64)
    return 2 * wide if 2 * wide <= cus else wide


# bench lines whose dominant kernel's HBM bytes are counted: workload, a
# substring of the kernel's name, the sources it is built from (counters
# taken on other source are not reported), and how one call is run
COUNTED = {
    "main": ("diag_bf16_b8_t4096_h16_d128", "kdn_chunk_kernel",
             ("kdn_chunked.hip", "kdn_device.h", "kdn_recurrent_core.h", "kdn_gates.h")),
    "isotropic": ("iso_bf16_b8_t4096_h16_d128", "kdn_iso_kernel", ("kdn_iso.hip", "kdn_device.h", "kdn_gates.h")),
    # the split forward's kernels (Mobius pre-pass, chunked segments, state
    # chaining, output correction): bytes per call
    "long_context": ("diag_bf16_b1_t65536_h16_d128", "kdn_",
                     ("kdn_chunked.hip", "kdn_split.hip", "kdn_device.h", "kdn_recurrent_core.h", "kdn_gates.h")),
    "decode": ("decode_diag_bf16_n256_h16_d128_s1024", "kdn_recurrent_kernel",
               ("kdn_recurrent.hip", "kdn_recurrent_core.h", "kdn_device.h", "kdn_gates.h")),
    "decode_isotropic": ("decode_iso_bf16_n256_h16_d128_s1024", "kdn_recurrent_kernel",
                         ("kdn_recurrent.hip", "kdn_recurrent_core.h", "kdn_device.h", "kdn_gates.h")),
    # the backward's kernels (uncertainty adjoint, memory adjoint, d c0): the
    # counters pass runs no other library kernel
    "backward": ("diag_bf16_b8_t4096_h16_d128", "kdn_", ("kdn_backward.hip", "kdn_backward_chunk.hip",
                                                          "kdn_chunked.hip", "kdn_device.h",
                                                          "kdn_recurrent_core.h", "kdn_gates.h")),
}


def segments_of(kdn, w) -> int:
    """Segments the split forward cuts w's sequences into on this device."""
    return kdn.forward_split_segments(w.B, w.T, w.H, w.dk, w.dv)


def kernel_source_hash(line: str = "main") -> str:
    """Hash of the sources of a counted line's kernel: HBM counters taken on
    other source are not reported."""
    h = hashlib.sha256()
    for name in COUNTED[line][2]:
        with open(os.path.join(ROOT, "kalman_delta_network_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(line: str, algo: str = "auto"):
    """Counted HBM bytes per call of a line's kernel, or None when there is no
    entry taken on the current source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        tr = json.load(f)
    ent = tr.get(line + "/" + algo)
    if ent and ent.get("kernel_hash") == kernel_source_hash(line):
        return ent["bytes_per_launch"]
    return None


def upload(x, dtype, dev):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    names = ("q", "k", "v", "z_alpha", "z_omega", "z_r") if "z_alpha" in x else ("q", "k", "v", "alpha", "omega", "r")
    out = {n: torch.from_numpy(x[n]).to(tdt).to(dev) for n in names}
    out["c0"] = torch.from_numpy(x["c0"]).to(dev)
    return out


WARM_SECONDS = 0.3  # minimum busy time before timing: the GPU clock ramps over tens of ms


def warm(fn, count, seconds=WARM_SECONDS):
    """Run fn `count` times, then keep running it until the GPU has been busy
    for `seconds` (a few steps alone leave the clock below its sustained
    level; measured: ~350 us per forward launch in the first ~20 ms against
    ~297 us afterwards).  Returns the number of calls made."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < count or time.perf_counter() - t0 < seconds:
        for _ in range(max(1, count)):
            fn()
            n += 1
        torch.cuda.synchronize()
    return n


def time_forward(kdn, w, t, steps, warmup, algo):
    """Returns (ms per step over the timed loop, mean single-launch ms).
    Inputs holding z_alpha, z_omega, z_r run the gated forward."""
    import torch
    out = (torch.empty((w.B, w.T, w.H, w.dv), dtype=t["q"].dtype, device=t["q"].device),
           torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=t["q"].device),
           torch.empty({"diagonal": (w.B, w.H, w.dk), "grouped": (w.B, w.H, w.rgroups, w.dk)}.get(w.variant, (w.B, w.H)),
                       dtype=torch.float32, device=t["q"].device))
    if "z_alpha" in t:
        def call():
            kdn.forward_gated(**t, mu=w.mu, variant=w.variant, algo=algo, out=out)
    elif algo == "split":
        ws = torch.empty(max(1, kdn.forward_split_workspace_size(w.B, w.T, w.H, w.dk, w.dv)), dtype=torch.uint8,
                         device=t["q"].device)

        def call():
            kdn.forward_split(**t, mu=w.mu, workspace=ws, out=out)
    else:
        def call():
            kdn.forward(**t, mu=w.mu, variant=w.variant, algo=algo, out=out)
    warm(call, warmup)
    # whole timed loop
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    # per-launch durations (events on the same stream the kernel runs on).
    # One untimed call first keeps the device busy while the host enqueues
    # the first timed launch; after the synchronisation above the device
    # would otherwise sit idle inside that interval for the host's launch
    # latency.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    call()
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms_launch = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return ms_step, ms_launch


def bench_decode(kdn, w, dev, steps_cap=None, gated=False, warm_up=True):
    """Time w.decode_steps consecutive kdn_step calls (tokens pre-uploaded);
    ``gated``: kdn_step_gated on gate pre-activations; ``warm_up``: first
    run steps on a scratch copy of the state until the clock has ramped."""
    import torch
    from kalman_delta_network_amd import workloads as wl
    nsteps = w.decode_steps if steps_cap is None else min(steps_cap, w.decode_steps)
    st = wl.decode_state(w)
    S = torch.from_numpy(st["S0"]).to(dev)
    p = torch.from_numpy(st["p0"]).to(dev)
    toks = []
    for s in range(nsteps):
        tok = wl.gated_decode_tokens(w, s) if gated else wl.decode_tokens(w, s)
        toks.append(upload(dict(tok, c0=np.ones(1, np.float32)), w.dtype, dev))
    o = torch.empty((w.B, w.H, w.dv), dtype=toks[0]["q"].dtype, device=dev)
    if gated:
        names = ("q", "k", "v", "z_alpha", "z_omega", "z_r")
        step = lambda tk, S_, p_: kdn.step_gated(**{n: tk[n] for n in names}, mu=w.mu, S=S_, p=p_, o=o)
    else:
        names = ("q", "k", "v", "alpha", "omega", "r")
        step = lambda tk, S_, p_: kdn.step(**{n: tk[n] for n in names}, mu=w.mu, S=S_, p=p_, variant=w.variant,
                                           o=o)
    if warm_up:
        S2, p2 = S.clone(), p.clone()  # warm-up on a scratch copy of the state
        warm(lambda: step(toks[0], S2, p2), 3)
        del S2, p2
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(nsteps):
        step(toks[s], S, p)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    return {"workload": w.name, "steps": nsteps, "ms_per_step": ms / nsteps,
            "tokens_per_s": w.B * nsteps / (ms / 1e3),
            "hbm_gbs_algorithmic": step_bytes(w) / (ms / nsteps / 1e3) / 1e9,
            "hbm_frac": step_bytes(w) / (ms / nsteps / 1e3) / 1e9 / HBM_PEAK_GBS}


def bench_varlen(kdn, dev, steps, algo):
    """Time the packed serving batch: 32 sequences of 256..1792 tokens (16
    heads, d = 128, diagonal bf16) in one kdn_forward_varlen call, scheduled
    longest first."""
    import torch
    from kalman_delta_network_amd import workloads as wl
    w = wl.VARLEN
    lengths = wl.varlen_lengths(w.seed, w.B, *wl.VARLEN_RANGE)
    x = wl.varlen_inputs(w, lengths)
    t = upload(x, w.dtype, dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    order = torch.from_numpy(kdn.longest_first(x["cu_seqlens"])).to(dev)  # schedule the longest first
    total = int(x["cu_seqlens"][-1])
    out = (torch.empty((total, w.H, w.dv), dtype=t["q"].dtype, device=dev),
           torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev),
           torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device=dev))
    call = lambda: kdn.forward_varlen(**t, cu_seqlens=cu, mu=w.mu, variant=w.variant, algo=algo, out=out,
                                      order=order)
    warm(call, 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = varlen_bytes(w, total)
    return {"workload": w.name, "sequences": w.B, "tokens": total,
            "lengths": [int(lengths.min()), int(lengths.max())], "ms_per_step": ms,
            "tokens_per_s": total / (ms / 1e3), "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}


def backward_call(kdn, w, dev, gated=False):
    """(call, workspace): one kdn_backward call (``gated``: kdn_backward_gated
    on gate pre-activations) on workload w with cotangent dO only."""
    import torch
    from kalman_delta_network_amd import workloads as wl
    t = upload(wl.gated_inputs(w) if gated else wl.forward_inputs(w), w.dtype, dev)
    dO = torch.from_numpy(wl.backward_cotangents(w, with_state=False)["dO"]).to(t["q"].dtype).to(dev)
    if gated:
        ws = torch.empty(kdn.backward_gated_workspace_size(w.B, w.T, w.H, w.dk, w.dv, w.variant, t["q"].dtype),
                         dtype=torch.uint8, device=dev)
        call = lambda: kdn.backward_gated(**t, mu=w.mu, dO=dO, variant=w.variant, workspace=ws)
    else:
        # the smallest workspace kdn_backward accepts for this variant and dtype
        ws = torch.empty(kdn.backward_workspace_size(w.B, w.T, w.H, w.dk, w.dv, w.variant, t["q"].dtype),
                         dtype=torch.uint8, device=dev)
        call = lambda: kdn.backward(**t, mu=w.mu, dO=dO, variant=w.variant, workspace=ws)
    return call, ws


def bench_backward(kdn, w, dev, steps, gated=False):
    """Time kdn_backward (``gated``: kdn_backward_gated) on workload w, inputs
    resident."""
    import torch
    call, ws = backward_call(kdn, w, dev, gated)
    warm(call, 1)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    return {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
            "hbm_frac": backward_bytes(w) / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "workspace_bytes": int(ws.numel())}


COPY_BYTES = 512 << 20  # calibration copy for the HBM byte counters
PER_CALL = ("backward", "long_context")  # lines of several kernels: bytes per call
PER_CALL_RUNS = 4  # calls in their counters pass


def counters_pass(args):
    """Workload for the rocprofv3 counter runs of one counted line: one
    device-to-device copy of COPY_BYTES (the calibration kernel), then three
    calls of the line (decode: 16 steps)."""
    import torch
    import kalman_delta_network_amd as kdn
    from kalman_delta_network_amd import workloads as wl
    dev = torch.device("cuda:0")
    kdn.load_library()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    line = args.counters_pass
    w = wl.WORKLOADS[COUNTED[line][0]]
    if line.startswith("decode"):
        bench_decode(kdn, w, dev, 16, warm_up=False)
    elif line == "backward":
        call, _ = backward_call(kdn, w, dev)
        for _ in range(PER_CALL_RUNS):
            call()
    elif line == "long_context":
        t = upload(wl.forward_inputs(w), w.dtype, dev)
        ws = torch.empty(max(1, kdn.forward_split_workspace_size(w.B, w.T, w.H, w.dk, w.dv)), dtype=torch.uint8,
                         device=dev)
        for _ in range(PER_CALL_RUNS):
            kdn.forward_split(**t, mu=w.mu, workspace=ws)
    else:
        t = upload(wl.forward_inputs(w), w.dtype, dev)
        for _ in range(3):
            kdn.forward(**t, mu=w.mu, variant=w.variant, algo=args.algo)
    torch.cuda.synchronize()
    print("counters pass done", flush=True)


def _read_counter_csv(run_dir, counter):
    """{dispatch id: (kernel name, value)} from a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    rows = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                d = r.get("Dispatch_Id") or r.get("Correlation_Id")
                rows[d] = (r.get("Kernel_Name", ""), rows.get(d, ("", 0.0))[1] + float(r["Counter_Value"]))
    return rows


def traffic_from(fetch_dir, write_dir, out_path, algo, line):
    """HBM bytes per launch of a counted line's kernel from FETCH_SIZE /
    WRITE_SIZE (KiB per dispatch), each scaled by the same counter of the
    calibration copy.  The backward's and the split forward's bytes are per
    call (the sum over their kernels' dispatches, divided by the number of
    calls)."""
    res = {}
    kname = COUNTED[line][1]
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counter_csv(run_dir, counter)
        copies = [v for n, v in rows.values() if "kdn" not in n and v > 0]
        hits = [v for n, v in rows.values() if kname in n]
        if not copies or not hits:
            raise SystemExit(f"{counter}: no calibration copy or {kname} dispatch in {run_dir}")
        scale = COPY_BYTES / (max(copies) * 1024.0)  # bytes per counted byte
        per = float(np.sum(hits)) / PER_CALL_RUNS if line in PER_CALL else float(np.mean(hits))
        res[counter] = {"kib_per_launch": per, "dispatches": len(hits), "copy_kib": max(copies), "scale": scale,
                        "bytes_per_launch": per * 1024.0 * scale}
    entry = {"workload": COUNTED[line][0], "kernel": kname, "kernel_hash": kernel_source_hash(line), "algo": algo,
             "bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"],
             "counters": res}
    data = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            data = json.load(f)
    data.pop(MAIN + "/" + algo, None)  # entries keyed by workload name predate the per-line keys
    data[line + "/" + algo] = entry
    with open(out_path, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(entry))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x):
    """The fp64 oracle on the host: the whole workload on all its OpenMP
    threads (one (batch, head) pair per thread at a time), then the first
    two batch rows on one thread."""
    import oracle
    fn = oracle.forward_diag if w.variant == "diagonal" else oracle.forward_iso
    names = ("q", "k", "v", "alpha", "omega", "r")
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    fn(**{n: x[n] for n in names}, c0=x["c0"], mu=w.mu)
    dt = time.perf_counter() - t0
    nb = min(2, w.B)
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        fn(**{n: x[n][:nb] for n in names}, c0=x["c0"], mu=w.mu)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full {w.name} workload (B={w.B}, T={w.T}, H={w.H}), fp64, {dt:.1f} s wall "
                      f"on {threads} threads",
            "value_1thread": nb * w.T / dt1,
            "sample_1thread": f"batch rows 0..{nb - 1} of the same workload on 1 thread, {dt1:.1f} s wall",
            "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--algo", default="auto", choices=["auto", "recurrent", "chunked"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the isotropic, decode, packed-batch, per-channel-decay isotropic, grouped-noise, "
                         "long-context and backward lines")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--counters-pass", choices=sorted(COUNTED),
                    help="run the workload of the rocprofv3 counter runs of one bench line and exit")
    ap.add_argument("--traffic-from", nargs=3, metavar=("LINE", "FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc CSV runs of a line's counters pass into its traffic entry "
                         "and exit")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE)
    args = ap.parse_args()
    if args.traffic_from:
        line, fetch_dir, write_dir = args.traffic_from
        if line not in COUNTED:
            raise SystemExit(f"unknown line {line}; counted lines: {sorted(COUNTED)}")
        traffic_from(fetch_dir, write_dir, args.traffic_out, args.algo, line)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(each (batch, head) pair is independent; see the sharding notes). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.counters_pass:
        counters_pass(args)
        return

    import torch
    import kalman_delta_network_amd as kdn
    from kalman_delta_network_amd import workloads as wl

    dev = torch.device("cuda:0")
    kdn.load_library()
    w = wl.WORKLOADS[MAIN]
    x = wl.forward_inputs(w)
    t = upload(x, w.dtype, dev)
    ms_step, ms_launch = time_forward(kdn, w, t, args.steps, args.warmup, args.algo)
    nbytes = forward_bytes(w)
    achieved = nbytes / (ms_launch / 1e3) / 1e9
    traffic = traffic_for("main", args.algo)
    extra = {}
    if not args.no_extra:
        wi = wl.WORKLOADS["iso_bf16_b8_t4096_h16_d128"]
        ti = upload(wl.forward_inputs(wi), wi.dtype, dev)
        mi, li = time_forward(kdn, wi, ti, max(3, args.steps // 2), 2, args.algo)
        extra["isotropic"] = {"workload": wi.name, "tokens_per_s": wi.B * wi.T / (mi / 1e3),
                              "ms_per_step": mi, "launch_ms": li, "algorithmic_bytes": forward_bytes(wi),
                              "hbm_frac": forward_bytes(wi) / (li / 1e3) / 1e9 / HBM_PEAK_GBS,
                              "traffic": traffic_for("isotropic", args.algo)}
        del ti
        extra["decode"] = bench_decode(kdn, wl.WORKLOADS["decode_diag_bf16_n256_h16_d128_s1024"], dev,
                                       args.decode_steps)
        extra["decode"]["traffic"] = traffic_for("decode")
        extra["decode_isotropic"] = bench_decode(kdn, wl.WORKLOADS["decode_iso_bf16_n256_h16_d128_s1024"], dev,
                                                 args.decode_steps)
        extra["decode_isotropic"]["traffic"] = traffic_for("decode_isotropic")
        # the same decode at N = 1024 sequences: a 1.07 GB state, four times the
        # 256 MB Infinity Cache, so the per-byte rate of this line is HBM's
        wd = wl.WORKLOADS["decode_diag_bf16_n256_h16_d128_s1024"].with_(name="decode_diag_bf16_n1024_h16_d128", B=1024)
        extra["decode_n1024"] = bench_decode(kdn, wd, dev, min(64, args.decode_steps or 64))
        extra["decode_gated"] = bench_decode(kdn, wl.WORKLOADS["decode_diag_bf16_n256_h16_d128_s1024"], dev,
                                             min(256, args.decode_steps or 256), gated=True)
        extra["varlen"] = bench_varlen(kdn, dev, max(3, args.steps // 2), args.algo)
        wc = wl.WORKLOADS["isoch_bf16_b8_t4096_h16_d128"]
        tc = upload(wl.forward_inputs(wc), wc.dtype, dev)
        mc, lc = time_forward(kdn, wc, tc, 3, 1, "auto")
        extra["isochannel"] = {"workload": wc.name, "tokens_per_s": wc.B * wc.T / (mc / 1e3), "ms_per_step": mc,
                               "hbm_frac": forward_bytes(wc) / (lc / 1e3) / 1e9 / HBM_PEAK_GBS}
        del tc
        wg = wl.WORKLOADS["grouped_bf16_b8_t4096_h16_d128"]
        tg = upload(wl.forward_inputs(wg), wg.dtype, dev)
        mg, lg = time_forward(kdn, wg, tg, 3, 1, "auto")
        extra["grouped"] = {"workload": wg.name, "tokens_per_s": wg.B * wg.T / (mg / 1e3), "ms_per_step": mg,
                            "hbm_frac": forward_bytes(wg) / (lg / 1e3) / 1e9 / HBM_PEAK_GBS}
        del tg
        tz = upload(wl.gated_inputs(w), w.dtype, dev)
        mz, lz = time_forward(kdn, w, tz, 3, 1, "auto")
        extra["gated"] = {"workload": w.name + " (gate pre-activations)", "tokens_per_s": w.B * w.T / (mz / 1e3),
                          "ms_per_step": mz, "hbm_frac": forward_bytes(w) / (lz / 1e3) / 1e9 / HBM_PEAK_GBS}
        del tz
        wiz = wl.WORKLOADS["iso_bf16_b8_t4096_h16_d128"]
        tz = upload(wl.gated_inputs(wiz), wiz.dtype, dev)
        mz, lz = time_forward(kdn, wiz, tz, 3, 1, "auto")
        extra["gated_isotropic"] = {"workload": wiz.name + " (gate pre-activations)",
                                    "tokens_per_s": wiz.B * wiz.T / (mz / 1e3), "ms_per_step": mz,
                                    "hbm_frac": forward_bytes(wiz) / (lz / 1e3) / 1e9 / HBM_PEAK_GBS}
        del tz
        wlc = wl.WORKLOADS["diag_bf16_b1_t65536_h16_d128"]
        tlc = upload(wl.forward_inputs(wlc), wlc.dtype, dev)
        mlc, llc = time_forward(kdn, wlc, tlc, 3, 1, "split")
        mlp, _ = time_forward(kdn, wlc, tlc, 2, 1, "auto")
        extra["long_context"] = {"workload": wlc.name, "algo": "split", "tokens_per_s": wlc.B * wlc.T / (mlc / 1e3),
                                 "ms_per_step": mlc, "launch_ms": llc, "algorithmic_bytes": forward_bytes(wlc),
                                 "hbm_frac": forward_bytes(wlc) / (llc / 1e3) / 1e9 / HBM_PEAK_GBS,
                                 "segments": segments_of(kdn, wlc),
                                 "ms_per_step_unsplit": mlp,
                                 "workgroups_unsplit": chunked_workgroups(
                                     wlc, torch.cuda.get_device_properties(dev).multi_processor_count),
                                 "traffic": traffic_for("long_context")}
        del tlc
        extra["backward"] = bench_backward(kdn, w, dev, 3)
        extra["backward"]["traffic"] = traffic_for("backward")
        extra["backward_gated"] = bench_backward(kdn, w, dev, 3, gated=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x)
    line = {
        "metric": "KDN forward tokens/sec at H=16,d_k=d_v=128 on 1 GPU; % of HBM/MFMA roofline",
        "value": w.B * w.T / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "variant": w.variant, "B": w.B, "T": w.T, "H": w.H, "d_k": w.dk,
                   "d_v": w.dv, "mu": w.mu, "state": "fp32", "algo": args.algo},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": nbytes, "launch_ms": ms_launch},
        "mfma": {"achieved": forward_flops(w) / (ms_launch / 1e3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": forward_flops(w) / (ms_launch / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                 "flops": forward_flops(w)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
