"""Throughput of chunked delta-rule prefill on one MI355X.

One step = one full prefill call (prep, scan and output kernels) over the
workload's inputs, already resident in HBM.  Every step is timed on its own
with HIP events on the launch stream; ms_per_step is the median.  The
roofline is priced against the published peaks and against the peaks this
GPU sustains in two microbenchmarks (libdrla_peaks.so: a streaming copy and
chains of dependent MFMAs).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline]

Workloads (seeded, synthetic): gdn_prefill (default: 1 x 4096 tokens,
16 heads, dk = dv = 128, bf16), kda_prefill, gdn_varlen, gdn_long, gdn_tiny.
gdn_decode / kda_decode time one decode step instead (256 sequences, one
token each, from a nonzero state), under their own metric; gdn_prefill_f16 /
kda_prefill_f16 are the prefill configs with fp16 q, k, v; ret_prefill /
gla_prefill run decay-only linear attention (no delta rule) at that shape.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN/KDA chunked-prefill tokens/s at H16 d128 T4096; % of MFMA/HBM roofline"
DECODE_METRIC = "GDN/KDA decode-step tokens/s (one token per sequence); % of HBM roofline"
DECAY_METRIC = "decay-only linear attention (RetNet/GLA form) chunked-prefill tokens/s; % of HBM roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 (and fp16) MFMA, published
F32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 MFMA, published
CHUNK = 64


def kernel_costs(spec, n_tokens, n_seqs):
    """Algorithmic bytes and flops per launch of each kernel.

    Bytes: the method's own tensors that the kernel reads or writes (q, k,
    v, beta, g, h0 in; o, ht out), never the workspace intermediates the
    two-kernel split adds -- so traffic above these figures is overhead of
    the design.  Flops: the MFMA work of the kernel counting full 16x16
    tiles as issued (the strictly-upper tiles of the 64x64 chunk products are
    skipped)."""
    es = 4 if spec.io == "f32" else 2
    dk, dv, hv, hqk = spec.dk, spec.dv, spec.h_v, spec.h_qk
    kda = spec.kind in ("kda", "gla")          # per-channel gate
    nb = 0 if spec.kind in ("ret", "gla") else 4  # beta bytes (decay-only: none)
    th = n_tokens * hv                         # token x value head
    tq = n_tokens * hqk                        # token x query/key head
    n_chunks = sum((L + CHUNK - 1) // CHUNK for L in spec.lens)
    ch = n_chunks * hv                         # (chunk, value head) units
    g_bytes = th * (dk if kda else 1) * 4
    state = n_seqs * hv * dk * dv * 4
    h0 = state if spec.h0_std > 0 else 0
    prep_b = 2 * tq * dk * es + th * nb + g_bytes
    scan_b = 2 * tq * dk * es + th * dv * es + (0 if kda else g_bytes) + h0 \
        + th * dv * es + state
    C = CHUNK
    tri = 10 * 16 * 16                          # lower 16x16 tiles of a 64x64 product
    prep_f = ch * 2 * (2 * tri * dk)            # K K^T and Q K^T
    scan_f = ch * 2 * (3 * C * dk * dv + 2 * 6 * 16 * 32 * dv)  # X, Q S, K~^T V'; Tb R, P V'
    return {"prep": (prep_b, prep_f), "scan": (scan_b, scan_f)}


def call_io_bytes(spec, n_tokens, n_seqs):
    """Algorithmic I/O of one whole call: q, k, v, beta, g and h0 (if any)
    in; o and ht out."""
    es = 4 if spec.io == "f32" else 2
    nbeta = 0 if spec.kind in ("ret", "gla") else 4
    return n_tokens * (2 * spec.h_qk * spec.dk * es + spec.h_v * spec.dv * es * 2 + spec.h_v * nbeta
                       + spec.h_v * (spec.dk if spec.kind in ("kda", "gla") else 1) * 4) \
        + (2 if spec.h0_std > 0 else 1) * n_seqs * spec.h_v * spec.dk * spec.dv * 4


class Hip:
    """Raw HIP events through libamdhip64 (the library records them on the
    stream its kernels run on)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


def kernel_source_hash():
    """sha256 over the HIP sources and headers of the library (not the
    peak microbenchmarks); a traffic figure measured on other sources no
    longer describes these kernels."""
    import hashlib
    csrc = os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")) and name != "drla_peaks.hip":
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic(kernel, workload):
    """HBM bytes per dispatch of `kernel` on `workload` from the committed
    rocprofv3 counter summary profiles/<kernel>_<workload>_traffic.md (lines
    "source_sha256: ..." and "hbm_bytes_per_dispatch: ..."), or None when
    there is none or it was measured on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip().strip("`*- ")] = val.strip().strip("`* ")
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


# Kernels each timed stage launches (the stage events bracket them all):
# prep = schedule and rank (packed input) and prep; scan = the scan, and
# when the call splits its sequences into segments the compose (more than
# two segments) and fix-up kernels, or the head-resident scan's transition,
# compose and value kernels.
STAGE_KERNELS = {"prep": ("schedule", "rank", "prep"), "scan": ("scan", "compose", "fix")}


def stage_traffic(stage, workload):
    """HBM bytes per call of a stage: the sum over its kernels' committed
    counter summaries, or None without one for the stage's main kernel."""
    if load_traffic(stage, workload) is None:
        return None
    parts = (load_traffic(k, workload) for k in STAGE_KERNELS.get(stage, (stage,)))
    return sum(p for p in parts if p is not None)


def _nmse(x, y):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = float((y * y).sum())
    return float(((x - y) ** 2).sum() / d) if d > 0 else float((x * x).sum())


def _rel_err(x, y):
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.abs(y).max()) if y.size else 0.0
    num = float(np.abs(x - y).max()) if y.size else 0.0
    return num / den if den > 0 else num


def _oracle_heads(oracle, x, spec, heads, threads):
    """The fp64 oracle over the listed value heads only (their q/k heads and
    gates with them)."""
    grp = spec.h_v // spec.h_qk
    hk = [h // grp for h in heads]
    q, k = x["q"][:, hk], x["k"][:, hk]
    v, g = x["v"][:, heads], x["g"][:, heads]
    h0 = None if x["h0"] is None else x["h0"][:, heads]
    cu = x["cu_seqlens"] if x["varlen"] else None
    if spec.kind in ("ret", "gla"):
        return oracle.recurrence_decay(q, k, v, g, h0, cu, per_channel=spec.kind == "gla")
    return oracle.recurrence(q, k, v, x["beta"][:, heads], g, h0, cu, kda=spec.kind == "kda",
                             threads=threads)


def cpu_baseline(x, spec, n_tokens, budget_s=10.0, o_gpu=None, ht_gpu=None):
    """The fp64 oracle on this host's cores over the whole workload, repeated
    until about `budget_s` of wall time, and on one core over a sample of
    heads.  Its first whole-workload result also gives the GPU result's
    error (NMSE and max-relative) on the bench workload.  Returns
    (cpu_baseline object, parity object or None)."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    decay = spec.kind in ("ret", "gla")
    units = spec.n_seqs * spec.h_v
    used = 1 if decay else min(cores, units)
    all_heads = list(range(spec.h_v))
    reps, t_total, first = 0, 0.0, None
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        res = _oracle_heads(oracle, x, spec, all_heads, cores)
        t_total += time.perf_counter() - t0
        reps += 1
        if first is None:
            first = res
        if reps == 1 and t_total > budget_s:
            break
    # one core: whole heads, one after another, for about a third of the budget
    h1, t1 = 0, 0.0
    while h1 < spec.h_v and (h1 == 0 or t1 < budget_s / 3):
        t0 = time.perf_counter()
        _oracle_heads(oracle, x, spec, [h1], 1)
        t1 += time.perf_counter() - t0
        h1 += 1
    one = n_tokens * h1 / spec.h_v / t1
    what = "decay-only token recurrence" if decay else "token recurrence"
    base = {"value": round(n_tokens * reps / t_total, 1), "unit": "tokens/s", "cores": used,
            "kind": "oracle",
            "sample": f"whole {spec.name} workload ({n_tokens} tokens x {spec.h_v} heads), "
                      f"fp64 {what}, {reps} run(s) in {t_total:.1f} s, "
                      + ("one thread" if decay else
                         f"threads over {units} (sequence, head) units on {cores} host cores"),
            "one_core": {"value": round(one, 1), "unit": "tokens/s", "cores": 1,
                         "sample": f"{h1} of {spec.h_v} heads of the workload, all tokens, one "
                                   f"thread, {t1:.1f} s, scaled to the whole workload"}}
    parity = None
    if o_gpu is not None:
        o_ref, ht_ref = first
        parity = {"vs": "fp64 oracle (token recurrence), whole bench workload",
                  "nmse_o": float(f"{_nmse(o_gpu, o_ref):.3e}"),
                  "nmse_ht": float(f"{_nmse(ht_gpu, ht_ref):.3e}"),
                  "rel_err_o": float(f"{_rel_err(o_gpu, o_ref):.3e}"),
                  "rel_err_ht": float(f"{_rel_err(ht_gpu, ht_ref):.3e}")}
    return base, parity


PEAKS_LIB = os.path.join(ROOT, "delta_rule_linear_chunked_amd", "_build", "libdrla_peaks.so")


def measure_peaks(torch, hip, stream, io):
    """Attainable peaks of this GPU: HBM bandwidth of a streaming copy (2 GiB
    read + 2 GiB written) and MFMA throughput
    of chains of dependent MFMAs in the workload's dtype (bf16 and fp16
    16x16x32, fp32 16x16x4).  Each figure is the mean of five launches
    after two untimed ones, timed with HIP events on `stream`."""
    if not os.path.exists(PEAKS_LIB):
        raise RuntimeError(f"{PEAKS_LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(PEAKS_LIB)
    lib.drla_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.drla_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int)]
    lib.drla_peak_mfma_grid.argtypes = [ctypes.c_int]
    dev = torch.device("cuda:0")
    e0, e1 = hip.event(), hip.event()
    sp = ctypes.c_void_p(stream)

    def timed(launch, n=5):
        launch()
        launch()
        hip.lib.hipEventRecord(ctypes.c_void_p(e0), sp)
        for _ in range(n):
            launch()
        hip.lib.hipEventRecord(ctypes.c_void_p(e1), sp)
        torch.cuda.synchronize()
        return hip.elapsed_ms(e0, e1) / n

    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def launch():
        rc = lib.drla_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                nbytes, sp)
        if rc != 0:
            raise RuntimeError(f"drla_peak_copy failed ({rc})")
    best_bw = 2 * nbytes / (timed(launch) * 1e-3) / 1e9
    torch.cuda.synchronize()
    if not torch.equal(dst[:: (1 << 20)], src[:: (1 << 20)]):
        raise RuntimeError("peak copy produced wrong data")
    del src, dst

    kind = {"bf16": 0, "f16": 1}.get(io, 2)
    iters = 2048 if kind == 2 else 4096
    grid = lib.drla_peak_mfma_grid(0)
    out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    flops = ctypes.c_double()

    def mlaunch():
        rc = lib.drla_peak_mfma(ctypes.c_void_p(out.data_ptr()), kind, iters, grid, sp,
                                ctypes.byref(flops), None)
        if rc != 0:
            raise RuntimeError(f"drla_peak_mfma failed ({rc})")
    ms = timed(mlaunch)
    tflops = flops.value / (ms * 1e-3) / 1e12
    hip.destroy(e0)
    hip.destroy(e1)
    return {"hbm_copy_gbs": round(best_bw, 1),
            "hbm_copy": "2 GiB read + 2 GiB written, one 16-byte non-temporal load and store "
                        "per thread",
            "mfma_tflops": round(tflops, 1),
            "mfma": f"{['bf16 16x16x32', 'fp16 16x16x32', 'fp32 16x16x4'][kind]}, 8 dependent "
                    f"chains per wave, {grid} workgroups of 4 waves, {iters} rounds"}


def copy_calibration(torch, dev, mib):
    """A plain elementwise copy of `mib` MiB (bf16 negate: reads and writes
    mib MiB), five times: the reference dispatch that scales the HBM byte
    counters of a rocprofv3 --pmc run."""
    if mib <= 0:
        return
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copy calibration: {n * 2} bytes read and {n * 2} bytes written per dispatch",
          file=sys.stderr)


def _pk(peaks, key):
    return None if peaks is None else peaks[key]


def _frac(achieved, peak, digits=4):
    return None if peak is None else round(achieved / peak, digits)


def timed_steps(torch, hip, stream, step, steps, stage_events):
    """Runs `steps` steps back to back on `stream`, each timed on its own:
    a HIP event at every step's start (with stage_events, the three events
    the library records at the start, between prep and scan, and at the end
    of the call), one after the last.  Returns (per-step ms, per-stage ms
    lists, host wall seconds).  A step's time runs from its start event to
    the next step's, so it includes whatever separates two calls."""
    sp = ctypes.c_void_p(stream)
    evs = [[hip.event() for _ in range(3 if stage_events else 1)] for _ in range(steps)]
    end = hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if stage_events:
            step(evs[i])
        else:
            hip.lib.hipEventRecord(ctypes.c_void_p(evs[i][0]), sp)
            step()
    hip.lib.hipEventRecord(ctypes.c_void_p(end), sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    starts = [e[0] for e in evs] + [end]
    per_step = [hip.elapsed_ms(starts[i], starts[i + 1]) for i in range(steps)]
    stages = {}
    if stage_events:
        stages = {"prep": [hip.elapsed_ms(e[0], e[1]) for e in evs],
                  "scan": [hip.elapsed_ms(e[1], e[2]) for e in evs]}
    for e in [x for es in evs for x in es] + [end]:
        hip.destroy(e)
    return per_step, stages, wall


def mean_step_ms(torch, hip, stream, step, steps):
    """Mean ms per step over `steps` back-to-back steps with no events
    between them (two events around the whole run)."""
    sp = ctypes.c_void_p(stream)
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), sp)
    for _ in range(steps):
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), sp)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(e0, e1) / steps
    hip.destroy(e0)
    hip.destroy(e1)
    return ms


def decode_bench(args, spec, x, torch, drla):
    """One decode step per timed step: every sequence's next token from the
    fixed state h0 (read) to a separate new state (written)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io = {"bf16": torch.bfloat16, "f16": torch.float16}.get(spec.io, torch.float32)
    q, k, v = (torch.from_numpy(x[n]).to(dev, io) for n in ("q", "k", "v"))
    beta = torch.from_numpy(x["beta"]).to(dev)
    g = torch.from_numpy(x["g"]).to(dev)
    h0 = torch.from_numpy(x["h0"]).to(dev)
    N = spec.n_seqs
    o = torch.empty((N, spec.h_v, spec.dv), dtype=io, device=dev)
    ht = torch.empty_like(h0)
    fn = drla.kda_decode if spec.kind == "kda" else drla.gdn_decode

    def step():
        fn(q, k, v, beta, g, h0, out=o, final_state=ht)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    ms_mean = mean_step_ms(torch, hip, stream, step, args.steps)
    per_step, _, wall = timed_steps(torch, hip, stream, step, args.steps, False)
    ms_step = statistics.median(per_step)
    peaks = None if args.no_peaks else measure_peaks(torch, hip, stream, spec.io)
    es = 4 if spec.io == "f32" else 2
    kda = spec.kind == "kda"
    # algorithmic bytes: q, k, v, beta, g, h0 in; o, new state out
    bytes_ = N * (2 * spec.h_qk * spec.dk * es + 2 * spec.h_v * spec.dv * es + spec.h_v * 4
                  + spec.h_v * (spec.dk if kda else 1) * 4) + 2 * N * spec.h_v * spec.dk * spec.dv * 4
    ach = bytes_ / (ms_step * 1e-3) / 1e9
    traffic = load_traffic("decode", spec.name)
    line = {
        "metric": DECODE_METRIC,
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.io,
        "data": "synthetic (seeded; q,k L2-normalised, v ~ N(0,1), beta = sigmoid(N(0,1)), "
                "log-gates uniform, state N(0, 0.02))",
        "config": {"workload": spec.name, "kind": spec.kind, "n_seqs": N, "tokens_per_seq": 1,
                   "h_qk": spec.h_qk, "h_v": spec.h_v, "dk": spec.dk, "dv": spec.dv,
                   "io": spec.io},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "peak_measured": _pk(peaks, "hbm_copy_gbs"),
                     "frac_measured": _frac(ach, _pk(peaks, "hbm_copy_gbs")), "kernel": "decode",
                     "traffic": traffic,
                     "traffic_gbs": None if traffic is None else
                     round(traffic / (ms_step * 1e-3) / 1e9, 1),
                     "kernel_ms": {"decode": round(ms_step, 5)},
                     "algorithmic_bytes_per_launch": int(bytes_)},
        "path": {"ms_per_step_mean_no_events": round(ms_mean, 5),
                 "ms_per_step_min": round(min(per_step), 5),
                 "ms_per_step_max": round(max(per_step), 5),
                 "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 4)},
        "peaks": peaks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity"] = cpu_baseline(
            x, spec, N, args.cpu_budget, o.float().cpu().numpy(), ht.float().cpu().numpy())
    copy_calibration(torch, dev, args.copy_calibration)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gdn_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak microbenchmarks (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the bench, run a plain elementwise copy of MIB MiB (bf16 negate: "
                         "reads and writes MIB MiB) five times, the reference dispatch that scales "
                         "the HBM byte counters of a rocprofv3 --pmc run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the prefill kernels "
              "shard by (sequence, head) with no collective, so run one process per GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import delta_rule_linear_chunked_amd as drla
    import workloads as W

    spec = W.spec_by_name(args.workload)
    x = W.make_inputs(spec)
    if args.workload in W.DECODE_WORKLOADS:
        return decode_bench(args, spec, x, torch, drla)
    n_tokens = int(x["cu_seqlens"][-1])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io = {"bf16": torch.bfloat16, "f16": torch.float16}.get(spec.io, torch.float32)
    q, k, v = (torch.from_numpy(x[n]).to(dev, io) for n in ("q", "k", "v"))
    beta = torch.from_numpy(x["beta"]).to(dev)
    g = torch.from_numpy(x["g"]).to(dev)
    h0 = None if x["h0"] is None else torch.from_numpy(x["h0"]).to(dev)
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev) if x["varlen"] else None
    cu_host = [int(c) for c in x["cu_seqlens"]] if x["varlen"] else None
    n_seqs = spec.n_seqs
    o = torch.empty((n_tokens, spec.h_v, spec.dv), dtype=io, device=dev)
    ht = torch.empty((n_seqs, spec.h_v, spec.dk, spec.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(max(drla.workspace_bytes(x["q"].shape, x["v"].shape, io, n_seqs, cu_host), 1),
                     dtype=torch.uint8, device=dev)
    if spec.kind in ("ret", "gla"):
        call = drla.prepare_prefill(spec.kind == "gla", q, k, v, None, g, h0, cu,
                                    cu_seqlens_host=cu_host, workspace=ws, out=o,
                                    final_state=ht, flags=drla.DECAY_ONLY)
    else:
        call = drla.prepare_prefill(spec.kind == "kda", q, k, v, beta, g, h0, cu,
                                    cu_seqlens_host=cu_host, workspace=ws, out=o,
                                    final_state=ht)

    # which scan the call takes (the library's own plan for these shapes)
    lay = drla.workspace_layout(x["q"].shape, x["v"].shape, io, n_seqs, cu_host,
                                kda=spec.kind in ("kda", "gla"),
                                flags=drla.DECAY_ONLY if spec.kind in ("ret", "gla") else 0)
    scan_form = ("head-resident" if lay.get("head_scan") else
                 "per-16-column, segment split" if lay["seg"] else "per-16-column, one pass")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    ms_mean = mean_step_ms(torch, hip, stream, call, args.steps)
    # the timed region: one event at every step's start, the median step;
    # then the same steps with the library's three stage events, the median
    # time of each stage (more events per step, so a separate run)
    per_step, _, wall = timed_steps(torch, hip, stream, call, args.steps, False)
    ms_step = statistics.median(per_step)
    _, stages, _ = timed_steps(torch, hip, stream, call, args.steps, True)
    stage = {kk: statistics.median(vv) for kk, vv in stages.items()}
    peaks = None if args.no_peaks else measure_peaks(torch, hip, stream, spec.io)

    costs = kernel_costs(spec, n_tokens, n_seqs)
    dom = max(stage, key=stage.get)
    bytes_, flops = costs[dom]
    t_s = stage[dom] * 1e-3
    intensity = flops / bytes_
    mfma_peak = F32_PEAK_TFLOPS if spec.io == "f32" else BF16_PEAK_TFLOPS
    ridge = mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        ach = bytes_ / t_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "peak_measured": _pk(peaks, "hbm_copy_gbs"),
                "frac_measured": _frac(ach, _pk(peaks, "hbm_copy_gbs"))}
    else:
        ach = flops / t_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(ach / mfma_peak, 4), "peak_measured": _pk(peaks, "mfma_tflops"),
                "frac_measured": _frac(ach, _pk(peaks, "mfma_tflops"))}
    roof["kernel"] = dom
    roof["traffic"] = stage_traffic(dom, spec.name)
    roof["stage_kernels"] = list(STAGE_KERNELS.get(dom, (dom,)))
    # HBM bytes per dispatch from the committed counter profiles (null when
    # they were taken on other kernel sources) over the live kernel times
    traffic_gbs = {}
    for kk in stage:
        tb = stage_traffic(kk, spec.name)
        traffic_gbs[kk] = None if tb is None else round(tb / (stage[kk] * 1e-3) / 1e9, 1)
    roof["traffic_gbs"] = traffic_gbs
    roof["kernel_ms"] = {kk: round(vv, 5) for kk, vv in stage.items()}
    roof["algorithmic_bytes_per_launch"] = int(bytes_)
    roof["algorithmic_flops_per_launch"] = int(flops)

    total_flops = sum(f for _, f in costs.values())
    io_bytes = call_io_bytes(spec, n_tokens, n_seqs)
    io_gbs = io_bytes / (ms_step * 1e-3) / 1e9
    path_tflops = total_flops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": DECAY_METRIC if spec.kind in ("ret", "gla") else METRIC,
        "value": round(n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.io,
        "data": "synthetic (seeded; q,k L2-normalised, v ~ N(0,1), beta = sigmoid(N(0,1)), "
                "log-gates uniform)",
        "config": {"workload": spec.name, "kind": spec.kind, "n_seqs": n_seqs,
                   "total_tokens": n_tokens, "h_qk": spec.h_qk, "h_v": spec.h_v,
                   "dk": spec.dk, "dv": spec.dv, "chunk": CHUNK, "io": spec.io},
        "roofline": roof,
        "path": {"algorithmic_io_bytes": int(io_bytes),
                 "io_roofline_frac": round(io_gbs / HBM_PEAK_GBS, 4),
                 "io_roofline_frac_measured": _frac(io_gbs, _pk(peaks, "hbm_copy_gbs")),
                 "kernel_flops": int(total_flops),
                 "mfma_frac": round(path_tflops / mfma_peak, 5),
                 "mfma_frac_measured": _frac(path_tflops, _pk(peaks, "mfma_tflops"), 5),
                 "ms_per_step_mean_no_events": round(ms_mean, 5),
                 "ms_per_step_min": round(min(per_step), 5),
                 "ms_per_step_max": round(max(per_step), 5),
                 "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
                 "scan_form": scan_form},
        "peaks": peaks,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity"] = cpu_baseline(
            x, spec, n_tokens, args.cpu_budget, o.float().cpu().numpy(), ht.float().cpu().numpy())
    copy_calibration(torch, dev, args.copy_calibration)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
