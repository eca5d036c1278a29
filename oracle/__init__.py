"""TEST INFRASTRUCTURE ONLY: the CPU oracle for delta-rule chunked prefill.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from this package.  The HIP product path
never imports, links or calls it, and the oracle shares no code with it:
the only common module is ``workloads`` (seeded random inputs, no arithmetic
of the method).

Two independent fp64 implementations live here:

``recurrence``  (C, ``recurrence.c``) -- the definition: the token-by-token
    gated delta rule of "Empowering Hybrid Attention Models on NPUs",
    Section 2.1 (state updated from K_t, V_t, then output read from the
    updated state with Q_t), GDN with a scalar gate and KDA with a
    per-channel gate.  This is the truth every GPU result is compared to.
    ``recurrence_decay`` (same file) is the decay-only form of RetNet and
    GLA that the page names in Section 8: no beta, no delta-rule erase.

``chunked``     (numpy, ``chunked.py``) -- the chunkwise Map-Reduce-Map
    evaluation the same page describes in Section 2.1 ("Chunkwise
    Map-Reduce-Map Execution": operators #1-#4 Gate, KKT, Solve, W/U; #5 H;
    #6 O).  It reaches the recurrence's result up to rounding and exposes
    every per-chunk intermediate.

Pins (tests/test_oracle_pins.py) tie both to facts that do not come from
either implementation: closed forms, invariants, and agreement between the
two independent algorithms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (in-tree, under oracle/_build)."""
    os.makedirs(_BUILD, exist_ok=True)
    src = os.path.join(_HERE, "recurrence.c")
    if force or not os.path.exists(_SO) or \
            os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread",
                               "-std=c99", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_SO)
            f = lib.oracle_delta_rule_f64
            dp = ctypes.POINTER(ctypes.c_double)
            f.argtypes = [ctypes.c_int, ctypes.c_int,
                          ctypes.POINTER(ctypes.c_int64),
                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                          ctypes.c_int, dp, dp, dp, dp, dp, dp, dp, dp,
                          ctypes.c_int]
            f.restype = ctypes.c_int
            f = lib.oracle_decay_f64
            f.argtypes = [ctypes.c_int, ctypes.c_int,
                          ctypes.POINTER(ctypes.c_int64),
                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                          ctypes.c_int, dp, dp, dp, dp, dp, dp, dp]
            f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrence(q, k, v, beta, g, h0=None, cu_seqlens=None, kda=False,
               threads: Optional[int] = None):
    """fp64 token-by-token recurrence.  Inputs are numpy arrays in the packed
    layouts q,k [T,h_qk,dk], v [T,h_v,dv], beta [T,h_v], g [T,h_v] (GDN) or
    [T,h_v,dk] (KDA), h0 [N,h_v,dk,dv] or None; cu_seqlens [N+1] or None
    (one sequence).  Returns (o [T,h_v,dv], ht [N,h_v,dk,dv]) in float64."""
    lib = _load()
    q, k, v, beta, g = map(_f64, (q, k, v, beta, g))
    T, h_qk, dk = q.shape
    _, h_v, dv = v.shape
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    h0a = None if h0 is None else _f64(h0)
    o = np.zeros((T, h_v, dv), dtype=np.float64)
    ht = np.zeros((n, h_v, dk, dv), dtype=np.float64)
    if threads is None:
        threads = len(os.sched_getaffinity(0))
    rc = lib.oracle_delta_rule_f64(
        int(bool(kda)), n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        h_qk, h_v, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(h0a), _ptr(o), _ptr(ht), int(threads))
    if rc != 0:
        raise ValueError("oracle: malformed arguments")
    return o, ht


def recurrence_decay(q, k, v, g, h0=None, cu_seqlens=None, per_channel=False):
    """fp64 token recurrence of decay-only linear attention (RetNet / GLA
    style, no delta rule: S_t = Diag(e^{g_t}) S_{t-1} + k_t v_t^T,
    o_t = S_t^T q_t).  Layouts as `recurrence`, without beta; g is
    [T, h_v] (scalar gate) or [T, h_v, dk] (per_channel).  Returns
    (o, ht) in float64."""
    lib = _load()
    q, k, v, g = map(_f64, (q, k, v, g))
    T, h_qk, dk = q.shape
    _, h_v, dv = v.shape
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else \
        np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    h0a = None if h0 is None else _f64(h0)
    o = np.zeros((T, h_v, dv), dtype=np.float64)
    ht = np.zeros((n, h_v, dk, dv), dtype=np.float64)
    rc = lib.oracle_decay_f64(
        int(bool(per_channel)), n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        h_qk, h_v, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0a), _ptr(o), _ptr(ht))
    if rc != 0:
        raise ValueError("oracle: malformed arguments")
    return o, ht


from .chunked import chunked  # noqa: E402  (numpy form, no C needed)

__all__ = ["recurrence", "recurrence_decay", "chunked", "build"]
