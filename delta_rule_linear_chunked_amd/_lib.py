"""ctypes binding of libdrla.so.  Names and argument order follow
include/drla.h; this module only converts torch tensors to pointers and
sizes, allocates outputs and the workspace with torch, and passes torch's
current HIP stream."""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "_build", "libdrla.so")
_lock = threading.Lock()
_lib = None

BF16, F32, F16 = 0, 1, 2
STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "unsupported size or dtype",
          4: "misaligned pointer", 5: "bad cu_seqlens", 6: "workspace too small",
          7: "overlapping buffers", 8: "HIP error"}


class DrlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"drla: {STATUS.get(status, status)}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64)]


class Layout(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in ("sched", "tb", "pm", "kt", "kw", "qw", "gam", "vp", "h",
                                       "seg", "hs", "total", "head_scan")]


KEEP_INTERMEDIATES = 1
DECAY_ONLY = 2
SERIAL = 4
HEAD_SCAN = 8
COLUMN_SCAN = 16


def lib_path() -> str:
    return _LIB


def load_library():
    """Load libdrla.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            raise RuntimeError(
                f"drla: {_LIB} is missing; build it with "
                "`python -m delta_rule_linear_chunked_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(_LIB)
        vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
        pp = ctypes.POINTER(Problem)
        for name in ("gdn_prefill", "kda_prefill"):
            f = getattr(lib, name)
            f.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp,
                          ctypes.c_size_t, vp]
            f.restype = ctypes.c_int
        for name in ("gdn_decode", "kda_decode"):
            f = getattr(lib, name)
            f.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            f.restype = ctypes.c_int
        lib.decay_prefill.argtypes = [ctypes.c_int, pp, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp,
                                      ctypes.c_size_t, vp]
        lib.decay_prefill.restype = ctypes.c_int
        lib.decay_decode.argtypes = [ctypes.c_int, pp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.decay_decode.restype = ctypes.c_int
        lib.drla_prefill_ex.argtypes = [ctypes.c_int, ctypes.c_int, pp, vp, vp, vp, vp, vp, vp,
                                        vp, i32p, vp, vp, vp, ctypes.c_size_t, vp,
                                        ctypes.POINTER(ctypes.c_void_p)]
        lib.drla_prefill_ex.restype = ctypes.c_int
        lib.drla_prefill_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, pp, vp, vp, vp, vp, vp, vp,
                                             vp, i32p, vp, vp, vp]
        lib.drla_prefill_noalloc.restype = ctypes.c_int
        lib.drla_prefill_status.argtypes = [pp, i32p, vp, vp]
        lib.drla_prefill_status.restype = ctypes.c_int
        lib.drla_workspace_bytes.argtypes = [pp, i32p]
        lib.drla_workspace_bytes.restype = ctypes.c_size_t
        lib.drla_workspace_layout.argtypes = [ctypes.c_int, pp, i32p, ctypes.c_int,
                                              ctypes.POINTER(Layout)]
        lib.drla_workspace_layout.restype = ctypes.c_int
        lib.drla_status_str.argtypes = [ctypes.c_int]
        lib.drla_status_str.restype = ctypes.c_char_p
        lib.drla_last_error.argtypes = []
        lib.drla_last_error.restype = ctypes.c_char_p
        lib.drla_version.argtypes = []
        lib.drla_version.restype = ctypes.c_int
        _lib = lib
        return lib


def _host_cu(cu_seqlens, cu_seqlens_host):
    if cu_seqlens is None:
        return None
    if cu_seqlens_host is None:
        cu_seqlens_host = cu_seqlens.cpu()  # synchronises; pass a host copy to avoid it
    if isinstance(cu_seqlens_host, torch.Tensor):
        arr = cu_seqlens_host.to(torch.int32).contiguous()
    else:
        arr = torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
    return arr


def _io_code(dtype):
    codes = {torch.bfloat16: BF16, torch.float32: F32, torch.float16: F16}
    if dtype not in codes:
        raise ValueError(f"q/k/v dtype must be bfloat16, float16 or float32, got {dtype}")
    return codes[dtype]


def _problem(q, v, n_seqs, total):
    if q.dtype != v.dtype:
        raise ValueError("q, k and v must have the same dtype")
    io = _io_code(q.dtype)
    return Problem(n_seqs, q.shape[-2], v.shape[-2], q.shape[-1], v.shape[-1], io, total)


def _i32p(t):
    if t is None:
        return None
    return ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))


def workspace_bytes(q_shape, v_shape, io_dtype=torch.bfloat16, n_seqs=1,
                    cu_seqlens_host: Optional[Sequence[int]] = None) -> int:
    """Workspace size in bytes for packed q [T,h_qk,dk] and v [T,h_v,dv]."""
    lib = load_library()
    T = q_shape[0]
    cu = None if cu_seqlens_host is None else torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
    if cu is not None:
        n_seqs = len(cu) - 1
    p = Problem(n_seqs, q_shape[1], v_shape[1], q_shape[2], v_shape[2],
                _io_code(io_dtype), T)
    return int(lib.drla_workspace_bytes(ctypes.byref(p), _i32p(cu)))


def workspace_layout(q_shape, v_shape, io_dtype=torch.bfloat16, n_seqs=1,
                     cu_seqlens_host: Optional[Sequence[int]] = None, kda: bool = False,
                     flags: int = 0) -> dict:
    """Workspace regions (byte offsets) of a drla_prefill_ex call with the
    same gate kind, shapes, lengths and flags."""
    lib = load_library()
    cu = None if cu_seqlens_host is None else torch.tensor(list(cu_seqlens_host), dtype=torch.int32)
    if cu is not None:
        n_seqs = len(cu) - 1
    p = Problem(n_seqs, q_shape[1], v_shape[1], q_shape[2], v_shape[2],
                _io_code(io_dtype), q_shape[0])
    out = Layout()
    st = lib.drla_workspace_layout(int(kda), ctypes.byref(p), _i32p(cu), int(flags),
                                   ctypes.byref(out))
    if st != 0:
        raise DrlaError(st, lib.drla_last_error().decode())
    return {n: getattr(out, n) for n, _ in Layout._fields_}


class PreparedPrefill:
    """One prefill call with its arguments validated and marshalled once;
    calling the object launches that call again (one C call) on the same
    buffers and stream, optionally with three stage events.  The tensors it
    was prepared from must stay alive and keep their storage."""

    def __init__(self, lib, kda, flags, args, o, ht, keep):
        self._lib, self._kda, self._flags, self._args = lib, int(kda), int(flags), args
        self._fn = lib.kda_prefill if kda else lib.gdn_prefill
        self.out, self.final_state = o, ht
        self._keep = keep  # the Problem struct, host lengths, workspace

    def __call__(self, stage_events=None, verify_lengths=False):
        if stage_events is not None or self._flags:
            evs = None if stage_events is None else (ctypes.c_void_p * 3)(*stage_events)
            st = self._lib.drla_prefill_ex(self._kda, self._flags, *self._args, evs)
        else:
            st = self._fn(*self._args)
        if st != 0:
            raise DrlaError(st, self._lib.drla_last_error().decode())
        if verify_lengths:
            self.check_lengths()
        return self.out, self.final_state

    def check_lengths(self):
        """drla_prefill_status of the last launch (waits for its stream):
        raises DrlaError if the device cu_seqlens differed from the host
        copy (the call then ran as empty sequences)."""
        a = self._args
        st = self._lib.drla_prefill_status(a[0], a[8], a[11], a[13])
        if st != 0:
            raise DrlaError(st, self._lib.drla_last_error().decode())


def _prefill(kda: bool, q, k, v, beta, g, initial_state=None, cu_seqlens=None,
             cu_seqlens_host=None, output_final_state=True, workspace=None,
             out=None, final_state=None, stage_events=None, flags=0, verify_lengths=False):
    return _prepare(kda, q, k, v, beta, g, initial_state, cu_seqlens, cu_seqlens_host,
                    output_final_state, workspace, out, final_state, flags)(stage_events,
                                                                            verify_lengths)


def prepare_prefill(kda: bool, q, k, v, beta, g, initial_state=None, cu_seqlens=None,
                    cu_seqlens_host=None, output_final_state=True, workspace=None,
                    out=None, final_state=None, flags=0) -> PreparedPrefill:
    """Validate and marshal one gdn_prefill (kda=False) or kda_prefill call
    (arguments as there; decay-only with flags=DECAY_ONLY and beta=None) on
    the current stream, without launching it.  Returns a PreparedPrefill;
    each call of it launches the prefill."""
    return _prepare(kda, q, k, v, beta, g, initial_state, cu_seqlens, cu_seqlens_host,
                    output_final_state, workspace, out, final_state, flags)


def _prepare(kda, q, k, v, beta, g, initial_state, cu_seqlens, cu_seqlens_host,
             output_final_state, workspace, out, final_state, flags):
    lib = load_library()
    decay = bool(flags & DECAY_ONLY)
    if q.dim() == 4:
        # dense batch [B, T, H, d]: B equal-length sequences
        if cu_seqlens is not None and q.shape[0] != 1:
            raise ValueError("with cu_seqlens, pass packed [T, H, d] inputs (or batch 1)")
        n_seqs = 1 if cu_seqlens is not None else q.shape[0]
        q, k, v = (x.reshape(-1, x.shape[-2], x.shape[-1]) for x in (q, k, v))
        if beta is not None:
            beta = beta.reshape(-1, beta.shape[-1])
        g = g.reshape(-1, *g.shape[2:])
    elif q.dim() == 3:
        n_seqs = 1
    else:
        raise ValueError("q must be [T, H, dk] or [B, T, H, dk]")
    cu_host = _host_cu(cu_seqlens, cu_seqlens_host)
    if cu_host is not None:
        n_seqs = cu_host.numel() - 1
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
    T = q.shape[0]
    for name, x in (("q", q), ("k", k), ("v", v), ("beta", beta), ("g", g)):
        if x is None and name == "beta" and decay:
            continue
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != q.shape or v.shape[0] != T:
        raise ValueError("q, k must be [T, h_qk, dk] and v [T, h_v, dv]")
    if (not decay and beta.dtype != torch.float32) or g.dtype != torch.float32:
        raise ValueError("beta and g must be float32")
    h_v, dk, dv = v.shape[1], q.shape[2], v.shape[2]
    want_g = (T, h_v, dk) if kda else (T, h_v)
    if (not decay and tuple(beta.shape) != (T, h_v)) or tuple(g.shape) != want_g:
        raise ValueError(f"beta must be {(T, h_v)} and g {want_g}")
    prob = _problem(q, v, n_seqs, T)
    dev = q.device
    if initial_state is not None:
        if initial_state.dtype != torch.float32 or not initial_state.is_contiguous() \
                or tuple(initial_state.shape) != (n_seqs, h_v, dk, dv):
            raise ValueError(f"initial_state must be contiguous float32 {(n_seqs, h_v, dk, dv)}")
    o = out if out is not None else torch.empty((T, h_v, dv), dtype=q.dtype, device=dev)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else \
            torch.empty((n_seqs, h_v, dk, dv), dtype=torch.float32, device=dev)
    if flags:
        lay = Layout()
        st = lib.drla_workspace_layout(int(kda), ctypes.byref(prob), _i32p(cu_host), int(flags),
                                       ctypes.byref(lay))
        if st != 0:
            raise DrlaError(st, lib.drla_last_error().decode())
        need = int(lay.total)
    else:
        need = int(lib.drla_workspace_bytes(ctypes.byref(prob), _i32p(cu_host)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
            None if beta is None else beta.data_ptr(), g.data_ptr(),
            None if initial_state is None else initial_state.data_ptr(),
            None if cu_seqlens is None else cu_seqlens.data_ptr(),
            _i32p(cu_host), o.data_ptr(), None if ht is None else ht.data_ptr(),
            workspace.data_ptr(), workspace.numel(), stream)
    return PreparedPrefill(lib, kda, flags, args, o, ht,
                           (prob, cu_host, workspace, q, k, v, beta, g, initial_state, cu_seqlens))


NOALLOC_SCRATCH_BYTES = 64 << 20  # DRLA_NOALLOC_SCRATCH_BYTES


def prefill_noalloc(kda: bool, q, k, v, beta, g, initial_state=None, cu_seqlens=None,
                    cu_seqlens_host=None, out=None, final_state=None, flags=0,
                    verify_lengths=False):
    """drla_prefill_noalloc: the prefill without a workspace argument (the
    library's own per-GPU scratch array serves instead).  Packed [T, H, d]
    inputs; o and the final state are allocated here unless `out` and
    `final_state` are given (the C call itself allocates nothing).  Returns
    (o, final_state)."""
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [T, H, dk]")
    cu_host = _host_cu(cu_seqlens, cu_seqlens_host)
    n_seqs = 1 if cu_host is None else cu_host.numel() - 1
    T, h_v, dk, dv = q.shape[0], v.shape[1], q.shape[2], v.shape[2]
    for name, x in (("q", q), ("k", k), ("v", v), ("g", g)):
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    prob = _problem(q, v, n_seqs, T)
    dev = q.device
    o = out if out is not None else torch.empty((T, h_v, dv), dtype=q.dtype, device=dev)
    ht = final_state if final_state is not None else \
        torch.empty((n_seqs, h_v, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.drla_prefill_noalloc(
        int(kda), int(flags), ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(),
        None if beta is None else beta.data_ptr(), g.data_ptr(),
        None if initial_state is None else initial_state.data_ptr(),
        None if cu_seqlens is None else cu_seqlens.data_ptr(), _i32p(cu_host),
        o.data_ptr(), ht.data_ptr(), stream)
    if st == 0 and verify_lengths:
        st = lib.drla_prefill_status(ctypes.byref(prob), _i32p(cu_host), None, stream)
    if st != 0:
        raise DrlaError(st, lib.drla_last_error().decode())
    return o, ht


def decay_prefill(q, k, v, g, initial_state=None, cu_seqlens=None, per_channel=None, **kw):
    """Decay-only linear attention (RetNet / GLA form, no delta rule):
    S_t = Diag(e^{g_t}) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.  g is [T, h_v]
    (scalar gate) or [T, h_v, dk] (per-channel; per_channel=None infers it
    from g's rank).  Other arguments and the result as gdn_prefill."""
    if per_channel is None:
        per_channel = g.dim() == q.dim()
    kw["flags"] = kw.get("flags", 0) | DECAY_ONLY
    return _prefill(bool(per_channel), q, k, v, None, g, initial_state, cu_seqlens, **kw)


def gdn_prefill(q, k, v, beta, g, initial_state=None, cu_seqlens=None, **kw):
    """Gated DeltaNet chunked prefill.  q,k [T,h_qk,dk] (or [B,T,h_qk,dk]),
    v [T,h_v,dv], beta [T,h_v] fp32, g [T,h_v] fp32 log-decay,
    initial_state [N,h_v,dk,dv] fp32 or None, cu_seqlens int32 [N+1] device
    tensor or None.  Returns (o [T,h_v,dv], final_state [N,h_v,dk,dv]).

    Keywords: cu_seqlens_host (the same lengths on the host; without it they
    are copied from the device, a synchronisation), output_final_state,
    workspace, out, final_state, flags, stage_events, verify_lengths (wait
    for the call and raise DrlaError if the device and host lengths
    differed, in which case it ran as empty sequences)."""
    return _prefill(False, q, k, v, beta, g, initial_state, cu_seqlens, **kw)


def kda_prefill(q, k, v, beta, g, initial_state=None, cu_seqlens=None, **kw):
    """Kimi Delta Attention chunked prefill; g is per key channel [T,h_v,dk]."""
    return _prefill(True, q, k, v, beta, g, initial_state, cu_seqlens, **kw)


def _decode(kda: bool, q, k, v, beta, g, state=None, out=None, final_state=None,
            in_place=False, decay=False):
    lib = load_library()
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError("q, k must be [N, h_qk, dk] and v [N, h_v, dv]")
    N, h_v, dk, dv = q.shape[0], v.shape[1], q.shape[2], v.shape[2]
    for name, x in (("q", q), ("k", k), ("v", v), ("beta", beta), ("g", g)):
        if x is None and name == "beta" and decay:
            continue
        if not x.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if (not decay and beta.dtype != torch.float32) or g.dtype != torch.float32:
        raise ValueError("beta and g must be float32")
    want_g = (N, h_v, dk) if kda else (N, h_v)
    if (not decay and tuple(beta.shape) != (N, h_v)) or tuple(g.shape) != want_g:
        raise ValueError(f"beta must be {(N, h_v)} and g {want_g}")
    if state is not None and (state.dtype != torch.float32 or not state.is_contiguous()
                              or tuple(state.shape) != (N, h_v, dk, dv)):
        raise ValueError(f"state must be contiguous float32 {(N, h_v, dk, dv)}")
    prob = _problem(q, v, N, N)
    dev = q.device
    o = out if out is not None else torch.empty((N, h_v, dv), dtype=q.dtype, device=dev)
    if in_place:
        if state is None:
            raise ValueError("in_place needs a state")
        ht = state
    else:
        ht = final_state if final_state is not None else \
            torch.empty((N, h_v, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if decay:
        st = lib.decay_decode(int(kda), ctypes.byref(prob), q.data_ptr(), k.data_ptr(),
                              v.data_ptr(), g.data_ptr(),
                              None if state is None else state.data_ptr(), o.data_ptr(),
                              ht.data_ptr(), stream)
    else:
        fn = lib.kda_decode if kda else lib.gdn_decode
        st = fn(ctypes.byref(prob), q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                g.data_ptr(), None if state is None else state.data_ptr(), o.data_ptr(),
                ht.data_ptr(), stream)
    if st != 0:
        raise DrlaError(st, lib.drla_last_error().decode())
    return o, ht


def gdn_decode(q, k, v, beta, g, state=None, **kw):
    """One Gated DeltaNet decode step: row n of q, k [N, h_qk, dk], v
    [N, h_v, dv], beta, g [N, h_v] is sequence n's next token; state
    [N, h_v, dk, dv] fp32 (None: zeros).  Returns (o [N, h_v, dv], new
    state); with in_place=True the state tensor is updated and returned."""
    return _decode(False, q, k, v, beta, g, state, **kw)


def kda_decode(q, k, v, beta, g, state=None, **kw):
    """One Kimi Delta Attention decode step; g is per key channel [N, h_v, dk]."""
    return _decode(True, q, k, v, beta, g, state, **kw)


def decay_decode(q, k, v, g, state=None, per_channel=None, **kw):
    """One decode step of decay-only linear attention (no beta); g [N, h_v]
    or [N, h_v, dk].  Result as gdn_decode."""
    if per_channel is None:
        per_channel = g.dim() == q.dim()
    return _decode(bool(per_channel), q, k, v, None, g, state, decay=True, **kw)
