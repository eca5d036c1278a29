"""The segment split of the register-fed scan (KDA in every io type, GDN and
decay-only with fp32 inputs).

A call whose scan leaves most of the chip idle splits every sequence's
chunks into np segments: segment 0 from the initial state, every later one
from zero and, by as many transition workgroups, from the identity with
V = 0; a compose kernel chains the states entering the segments and a
fix-up adds their contribution to the outputs.  Each case runs on a
workspace filled with NaN bytes (the split's first state set must have been
written, and nothing the call reads may be a leftover NaN) and is checked
against the oracle and against the one-pass scan of the same call
(DRLA_SERIAL).  Cases: 2 to 16 segments, ragged last chunks, grouped heads,
dk = 64 and 128, a dense batch, no initial state, no final state, packed
batches with short and empty sequences, per-channel strong gates."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

IO = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _per_channel(kind):
    return kind in ("kda", "gla")


def _flags(drla, kind):
    return drla.DECAY_ONLY if kind in ("ret", "gla") else 0


def _splits(drla, x, kind, n_seqs, cu_host=None):
    lay = drla.workspace_layout(x["q"].shape, x["v"].shape, IO[x["io"]], n_seqs=n_seqs,
                                cu_seqlens_host=cu_host, kda=_per_channel(kind),
                                flags=_flags(drla, kind))
    off = lay["seg"]
    return off != 0, lay["total"], (off, off + n_seqs * x["h_v"] * x["dk"] * x["dv"] * 4)


def _call(drla, kind, d, dense_batch, flags, want_ht, ws=None, cu_host=None):
    q, k, v, beta, g, h0 = d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"]
    cu = d["cu"] if cu_host is not None else None
    if dense_batch > 1:
        q, k, v = (t.view(dense_batch, -1, *t.shape[1:]) for t in (q, k, v))
        beta, g = (t.view(dense_batch, -1, *t.shape[1:]) for t in (beta, g))
    fn = drla.kda_prefill if _per_channel(kind) else drla.gdn_prefill
    return fn(q, k, v, None if kind in ("ret", "gla") else beta, g, h0, cu, cu_seqlens_host=cu_host,
              flags=flags | _flags(drla, kind), output_final_state=want_ht, workspace=ws)


# (kind, io, h_qk, h_v, d, lens, packed, h0_std, want_ht, g_hi)
CASES = [
    ("kda", "bf16", 1, 2, 128, (4096,), False, 0.05, True, 0.15),    # 8 segments
    ("kda", "bf16", 2, 4, 128, (1000,), False, 0.05, True, 0.15),    # 3 segments, ragged tail
    ("kda", "f16", 2, 2, 64, (2000,), False, 0.05, True, 0.15),      # 8 segments, d = 64
    ("kda", "f32", 1, 2, 128, (3000,), False, 0.0, True, 0.15),      # no initial state
    ("kda", "f32", 2, 2, 64, (777,), False, 0.05, False, 0.15),      # no final state
    ("kda", "bf16", 1, 1, 128, (4096,), False, 0.05, True, 8.0),     # 16 segments, strong gates
    ("kda", "bf16", 1, 2, 128, (600, 600), False, 0.05, True, 0.15),  # dense batch
    ("kda", "bf16", 1, 2, 128, (1500, 700, 0, 2100), True, 0.05, True, 0.15),  # packed
    ("kda", "f16", 1, 1, 128, (3000, 100, 0), True, 0.05, True, 0.15),         # packed, short
    ("gdn", "f32", 1, 2, 128, (3000,), False, 0.05, True, 0.2),      # GDN, fp32
    ("gdn", "f32", 2, 2, 64, (1500, 700), True, 0.05, True, 0.2),    # GDN, fp32, packed
    ("gla", "bf16", 1, 2, 128, (2500,), False, 0.05, True, 0.2),     # per-channel decay-only
    ("ret", "f32", 1, 2, 64, (1500,), False, 0.05, True, 0.2),       # scalar decay-only, fp32
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-h{c[3]}-d{c[4]}-{'x'.join(map(str, c[5]))}"
                                             f"{'-packed' if c[6] else ''}-g{c[9]}" for c in CASES])
def test_register_scan_segment_split(drla, case):
    kind, io, h_qk, h_v, dk, lens, packed, h0_std, want_ht, g_hi = case
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dk, io=io,
                        g_lo=0.01, g_hi=g_hi, h0_std=h0_std, seed=47, varlen=packed)
    x = W.make_inputs(spec)
    n = len(lens)
    cu_host = [int(c) for c in x["cu_seqlens"]] if packed else None
    splits, wsb, rng = _splits(drla, x, kind, n, cu_host)
    print(f"case register-scan segment kind={kind} io={io} h_v={h_v} d={dk} lens={lens} "
          f"packed={packed} ht={want_ht} splits={splits}", flush=True)
    assert splits, "the case is meant to split"
    d = to_device(x)
    ws = torch.full((max(wsb, 1),), 255, dtype=torch.uint8, device="cuda")
    dense = 1 if packed else n
    o, ht = _call(drla, kind, d, dense, 0, want_ht, ws, cu_host)
    o1, ht1 = _call(drla, kind, d, dense, drla.SERIAL, want_ht, None, cu_host)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ws[rng[0]:rng[1]].view(torch.float32)).all()), \
        "the split scan did not run"
    o, o1 = (t.reshape(-1, h_v, dk).float().cpu().numpy() for t in (o, o1))
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[io]
    eo, eo1 = rel_err(o, o_ref), rel_err(o1, o_ref)
    print(f"  rel_err o split={eo:.3e} one-pass={eo1:.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and eo <= tol and eo1 <= tol
    assert rel_err(o, o1) <= tol
    if want_ht:
        ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
        eh = rel_err(ht, ht_ref)
        print(f"  rel_err ht split={eh:.3e} one-pass={rel_err(ht1, ht_ref):.3e}", flush=True)
        assert np.isfinite(ht).all() and eh <= tol
    else:
        assert ht is None and ht1 is None


def test_register_scan_split_repeatable(drla):
    """Two calls of the split KDA scan agree bit for bit."""
    spec = W.small_spec("kda", lens=(4000,), h_qk=1, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.15, h0_std=0.05, seed=48)
    d = to_device(W.make_inputs(spec))
    a = drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    b = drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
