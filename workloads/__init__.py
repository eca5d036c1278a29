"""Seeded synthetic inputs for delta-rule chunked prefill.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic, so both the fp64 oracle and the
HIP path may use it without sharing any computation.

The named workloads follow the shapes and value distributions that the
"Empowering Hybrid Attention Models on NPUs" page evaluates (Section 7.1:
chunk size 64, 16-bit Q/K/V, fp32 gates and states, 4,096-token prefill,
up to 65,536 tokens in Section 7.5).  Draw order is fixed: sequence lengths
(varlen only), q, k, v, beta, g, h0 -- all in float64 before any cast.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

__all__ = ["Spec", "WORKLOADS", "make_inputs", "bf16_round", "bf16_bits",
           "spec_by_name"]


@dataclass(frozen=True)
class Spec:
    """One synthetic prefill problem.

    kind      "gdn" (scalar log-gate per token and v-head) or "kda"
              (per-channel log-gate per token, v-head and key channel);
              "ret" / "gla": decay-only linear attention (no delta rule;
              beta is drawn but unused) with a scalar / per-channel gate.
    lens      sequence lengths; a packed batch uses cu_seqlens.
    h_qk/h_v  query/key heads and value heads; v-head h reads q/k head
              h // (h_v // h_qk).
    io        "bf16", "f16" or "f32": storage type of q, k, v (and o).
    g_lo/g_hi the log-gate is drawn as -U(g_lo, g_hi).
    h0_std    0 for a zero initial state, else N(0, h0_std) per element.
    varlen    True to pass cu_seqlens even for one sequence.
    """
    name: str
    kind: str
    lens: tuple
    h_qk: int
    h_v: int
    dk: int
    dv: int
    io: str
    g_lo: float
    g_hi: float
    h0_std: float = 0.0
    varlen: bool = False
    seed: int = 0
    random_lens: Optional[tuple] = None  # (count, lo, hi) drawn first

    @property
    def n_seqs(self) -> int:
        return len(self.lens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lens))


def _draw_lens(seed: int, count: int, lo: int, hi: int) -> tuple:
    rng = np.random.default_rng(seed)
    return tuple(int(x) for x in rng.integers(lo, hi, size=count, endpoint=True))


# The five workloads.  Index = seed.
WORKLOADS = {
    "gdn_tiny": Spec("gdn_tiny", "gdn", (256,), 2, 2, 64, 64, "f32",
                     0.01, 0.2, 0.0, seed=0),
    "gdn_prefill": Spec("gdn_prefill", "gdn", (4096,), 16, 16, 128, 128,
                        "bf16", 0.01, 0.2, 0.0, seed=1),
    "kda_prefill": Spec("kda_prefill", "kda", (4096,), 16, 16, 128, 128,
                        "bf16", 0.005, 0.15, 0.02, seed=2),
    "gdn_varlen": Spec("gdn_varlen", "gdn", _draw_lens(3, 8, 512, 8192),
                       16, 32, 128, 128, "bf16", 0.01, 0.2, 0.02,
                       varlen=True, seed=3, random_lens=(8, 512, 8192)),
    "gdn_long": Spec("gdn_long", "gdn", (65536,), 32, 32, 128, 128, "bf16",
                     0.001, 0.05, 0.02, seed=4),
}

# Decode steps (one token per sequence from a nonzero state): a serving
# batch of 256 sequences at the prefill configs' head shape.
DECODE_WORKLOADS = {
    "gdn_decode": Spec("gdn_decode", "gdn", (1,) * 256, 16, 16, 128, 128, "bf16",
                       0.01, 0.2, 0.02, varlen=True, seed=5),
    "kda_decode": Spec("kda_decode", "kda", (1,) * 256, 16, 16, 128, 128, "bf16",
                       0.005, 0.15, 0.02, varlen=True, seed=6),
}


# The prefill configs with fp16 q, k, v (the precision of the pages'
# experiment setup).
F16_WORKLOADS = {
    "gdn_prefill_f16": Spec("gdn_prefill_f16", "gdn", (4096,), 16, 16, 128, 128,
                            "f16", 0.01, 0.2, 0.0, seed=1),
    "kda_prefill_f16": Spec("kda_prefill_f16", "kda", (4096,), 16, 16, 128, 128,
                            "f16", 0.005, 0.15, 0.02, seed=2),
}


# Decay-only linear attention at the prefill configs' shape (the RetNet /
# GLA form: scalar and per-channel gates).
DECAY_WORKLOADS = {
    "ret_prefill": Spec("ret_prefill", "ret", (4096,), 16, 16, 128, 128, "bf16",
                        0.01, 0.2, 0.02, seed=7),
    "gla_prefill": Spec("gla_prefill", "gla", (4096,), 16, 16, 128, 128, "bf16",
                        0.005, 0.15, 0.02, seed=8),
}


# Long-context prefill with few heads per GPU: one 65,536-token sequence
# with 2 value heads (16 heads sharded over 8 GPUs by head), d = 128.
FEW_HEAD_WORKLOADS = {
    "gdn_long_h2": Spec("gdn_long_h2", "gdn", (65536,), 2, 2, 128, 128, "bf16",
                        0.001, 0.05, 0.02, seed=9),
    "kda_long_h2": Spec("kda_long_h2", "kda", (65536,), 2, 2, 128, 128, "bf16",
                        0.001, 0.05, 0.02, seed=10),
}


def spec_by_name(name: str) -> Spec:
    for table in (WORKLOADS, DECODE_WORKLOADS, F16_WORKLOADS, DECAY_WORKLOADS, FEW_HEAD_WORKLOADS):
        if name in table:
            return table[name]
    raise KeyError(name)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); returned
    as float32 holding exactly representable values.  NaN/Inf are not
    expected in these inputs."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return bits.view(np.float32)


def f16_round(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest IEEE half (ties to even), returned
    as float32 holding exactly representable values (inputs here are far
    inside the half range)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values already representable in bfloat16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # L2-normalise along the last axis (per token-head), as the workloads
    # specify for q and k.  Pure input preparation, not the method.
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return x / n


def make_inputs(spec: Spec, seed: Optional[int] = None) -> dict:
    """Draw one problem.  Returns numpy arrays:

    q, k   [T, h_qk, dk]   float32 (bf16- / fp16-representable when io is
                           "bf16" / "f16")
    v      [T, h_v, dv]    float32 (same)
    beta   [T, h_v]        float32, sigmoid(N(0,1))
    g      [T, h_v] or [T, h_v, dk]  float32 log-decay, -U(g_lo, g_hi)
    h0     [N, h_v, dk, dv] float32 or None
    cu_seqlens [N+1] int32
    """
    seed = spec.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = spec.lens
    if spec.random_lens is not None:
        cnt, lo, hi = spec.random_lens
        lens = tuple(int(x) for x in rng.integers(lo, hi, size=cnt, endpoint=True))
    T = int(sum(lens))
    q = _unit_rows(rng.standard_normal((T, spec.h_qk, spec.dk)))
    k = _unit_rows(rng.standard_normal((T, spec.h_qk, spec.dk)))
    v = rng.standard_normal((T, spec.h_v, spec.dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, spec.h_v))))
    gshape = (T, spec.h_v) if spec.kind in ("gdn", "ret") else (T, spec.h_v, spec.dk)
    g = -rng.uniform(spec.g_lo, spec.g_hi, size=gshape)
    h0 = None
    if spec.h0_std > 0:
        h0 = (spec.h0_std * rng.standard_normal(
            (len(lens), spec.h_v, spec.dk, spec.dv))).astype(np.float32)
    if spec.io == "bf16":
        cast = bf16_round
    elif spec.io == "f16":
        cast = f16_round
    else:
        cast = lambda a: a.astype(np.float32)  # noqa: E731
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return dict(q=cast(q), k=cast(k), v=cast(v),
                beta=beta.astype(np.float32), g=g.astype(np.float32), h0=h0,
                cu_seqlens=cu, lens=tuple(lens), kind=spec.kind, io=spec.io,
                h_qk=spec.h_qk, h_v=spec.h_v, dk=spec.dk, dv=spec.dv,
                varlen=spec.varlen or len(lens) > 1)


def small_spec(kind="gdn", lens=(200,), h_qk=2, h_v=2, dk=64, dv=64,
               io="f32", g_lo=0.01, g_hi=0.2, h0_std=0.0, seed=0,
               varlen=None) -> Spec:
    """A small ad-hoc problem for tests."""
    if varlen is None:
        varlen = len(lens) > 1
    return Spec(f"small_{kind}", kind, tuple(lens), h_qk, h_v, dk, dv, io,
                g_lo, g_hi, h0_std, varlen=varlen, seed=seed)
