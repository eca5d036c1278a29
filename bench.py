"""Throughput of chunked delta-rule prefill on one MI355X.

One step = one full prefill call (prep, scan and output kernels) over the
workload's inputs, already resident in HBM.  Prints one JSON line.

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
    """sha256 over the HIP sources and headers of the library; a traffic
    figure measured on other sources no longer describes these kernels."""
    import hashlib
    csrc = os.path.join(ROOT, "delta_rule_linear_chunked_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
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


def cpu_baseline(x, spec, n_tokens, budget_s=10.0):
    """The fp64 oracle on this host's cores over the whole workload,
    repeated until about `budget_s` of wall time."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    if spec.kind in ("ret", "gla"):
        # decay-only linear attention: the single-threaded fp64 recurrence
        reps, t_total = 0, 0.0
        while t_total < budget_s and reps < 1000:
            t0 = time.perf_counter()
            oracle.recurrence_decay(x["q"], x["k"], x["v"], x["g"], x["h0"],
                                    x["cu_seqlens"] if x["varlen"] else None,
                                    per_channel=spec.kind == "gla")
            t_total += time.perf_counter() - t0
            reps += 1
        return {"value": round(n_tokens * reps / t_total, 1), "unit": "tokens/s", "cores": 1,
                "kind": "oracle",
                "sample": f"whole {spec.name} workload ({n_tokens} tokens x {spec.h_v} heads), "
                          f"fp64 decay-only token recurrence, {reps} run(s) in {t_total:.1f} s, "
                          "one thread"}
    units = spec.n_seqs * spec.h_v
    used = min(cores, units)
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.recurrence(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"],
                          x["cu_seqlens"] if x["varlen"] else None,
                          kda=spec.kind == "kda", threads=cores)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps == 1 and t_total > budget_s:
            break
    return {"value": round(n_tokens * reps / t_total, 1), "unit": "tokens/s", "cores": used,
            "kind": "oracle",
            "sample": f"whole {spec.name} workload ({n_tokens} tokens x {spec.h_v} heads), "
                      f"fp64 token recurrence, {reps} run(s) in {t_total:.1f} s, "
                      f"threads over {units} (sequence, head) units on {cores} host cores"}


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
    e0, e1 = hip.event(), hip.event()
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
    for _ in range(args.steps):
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = hip.elapsed_ms(e0, e1) / args.steps
    hip.destroy(e0)
    hip.destroy(e1)
    es = 4 if spec.io == "f32" else 2
    kda = spec.kind == "kda"
    # algorithmic bytes: q, k, v, beta, g, h0 in; o, new state out
    bytes_ = N * (2 * spec.h_qk * spec.dk * es + 2 * spec.h_v * spec.dv * es + spec.h_v * 4
                  + spec.h_v * (spec.dk if kda else 1) * 4) + 2 * N * spec.h_v * spec.dk * spec.dv * 4
    ach = bytes_ / (ms_step * 1e-3) / 1e9
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
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": "decode",
                     "traffic": load_traffic("decode", spec.name),
                     "kernel_ms": {"decode": round(ms_step, 5)},
                     "algorithmic_bytes_per_launch": int(bytes_)},
        "path": {"host_wall_ms_per_step": round(wall * 1e3 / args.steps, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, spec, N, args.cpu_budget)
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
        def fn(q, k, v, beta, g, *a, **kw):
            return drla.decay_prefill(q, k, v, g, *a, per_channel=spec.kind == "gla", **kw)
    else:
        fn = drla.kda_prefill if spec.kind == "kda" else drla.gdn_prefill

    def step(events=None):
        fn(q, k, v, beta, g, h0, cu, cu_seqlens_host=cu_host, workspace=ws, out=o,
           final_state=ht, stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hip = Hip()
    e0, e1 = hip.event(), hip.event()
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.lib.hipEventRecord(ctypes.c_void_p(e0), ctypes.c_void_p(stream))
    for _ in range(args.steps):
        step()
    hip.lib.hipEventRecord(ctypes.c_void_p(e1), ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = hip.elapsed_ms(e0, e1)
    ms_step = ms_total / args.steps

    # per-kernel durations, live, with events at the stage boundaries
    stage = {"prep": 0.0, "scan": 0.0}
    evs = [hip.event() for _ in range(3)]
    for _ in range(args.steps):
        step(evs)
        torch.cuda.synchronize()
        stage["prep"] += hip.elapsed_ms(evs[0], evs[1])
        stage["scan"] += hip.elapsed_ms(evs[1], evs[2])
    for key in stage:
        stage[key] /= args.steps
    for e in evs + [e0, e1]:
        hip.destroy(e)

    costs = kernel_costs(spec, n_tokens, n_seqs)
    dom = max(stage, key=stage.get)
    bytes_, flops = costs[dom]
    t_s = stage[dom] * 1e-3
    intensity = flops / bytes_
    ridge = (F32_PEAK_TFLOPS if spec.io == "f32" else BF16_PEAK_TFLOPS) * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        ach = bytes_ / t_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = flops / t_s / 1e12
        peak = F32_PEAK_TFLOPS if spec.io == "f32" else BF16_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4)}
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom, spec.name)
    roof["kernel_ms"] = {kk: round(vv, 5) for kk, vv in stage.items()}
    roof["algorithmic_bytes_per_launch"] = int(bytes_)
    roof["algorithmic_flops_per_launch"] = int(flops)

    total_flops = sum(f for _, f in costs.values())
    io_bytes = call_io_bytes(spec, n_tokens, n_seqs)
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
                 "io_roofline_frac": round(io_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "kernel_flops": int(total_flops),
                 "mfma_frac": round(total_flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5),
                 "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, spec, n_tokens, args.cpu_budget)
    copy_calibration(torch, dev, args.copy_calibration)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
