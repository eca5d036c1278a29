"""The segment split of calls that leave most of the chip idle, in both
scans that have one.

Per-16-column scan (the default): segment 0 from the initial state, every
later one from zero and from the identity, then a compose and an output
fix-up; with 16 heads of d = 128 (too wide for that) the two chains of a
later segment share a workgroup and segment 0 is made longer than the rest.  Head-resident scan (DRLA_HEAD_SCAN): every sequence's chunks are
split into np segments; a transition kernel computes each segment's affine
state map (Phi, N) at once, a compose kernel chains the states entering the
segments, and the value kernel rescans every segment from its entering
state with the outputs.

Whether a call splits follows each scan's rule (the workspace layout
reports the split's region).  The cases take 2 to 16 segments, uneven last
segments, ragged last chunks, grouped heads, dk = 64 and 128, a dense batch,
no initial state, no final state, short and empty packed sequences and the
decay-only form; each is checked against the oracle and against the
one-pass scan of the same call (DRLA_SERIAL).  The split call runs on a
workspace filled with NaN bytes: when the rule splits it, the split's first
state set must have been written (and nothing the call reads may be a
leftover NaN); when it does not, the result equals one pass bit for bit."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


PATHS = ["head", "column"]


def _base(drla, path):
    return drla.HEAD_SCAN if path == "head" else 0


def _splits(drla, x, path, kind, n_seqs=1, cu_host=None):
    """(does the call split, workspace bytes, byte range of the split's first
    state set): the layout holds the split's region when it splits."""
    io = {"bf16": torch.bfloat16, "f16": torch.float16}[x["io"]]
    lay = drla.workspace_layout(x["q"].shape, x["v"].shape, io, n_seqs=n_seqs,
                                cu_seqlens_host=cu_host, kda=False,
                                flags=_base(drla, path) | (drla.DECAY_ONLY if kind == "ret" else 0))
    off = lay["hs" if path == "head" else "seg"]
    units = n_seqs * x["h_v"]
    return off != 0, lay["total"], (off, off + units * x["dk"] * x["dv"] * 4)


def _nan_workspace(nbytes):
    """A workspace whose every float reads NaN (bytes 0xFF)."""
    return torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device="cuda")


def _written(ws, rng):
    """The split wrote the first state set of its region: every float finite."""
    a, b = rng
    return bool(torch.isfinite(ws[a:b].view(torch.float32)).all())


def _call(drla, kind, d, dense_batch, flags, want_ht, ws=None):
    q, k, v, beta, g, h0 = d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"]
    if dense_batch > 1:
        q, k, v = (x.view(dense_batch, -1, *x.shape[1:]) for x in (q, k, v))
        beta, g = (x.view(dense_batch, -1, *x.shape[1:]) for x in (beta, g))
    if kind == "ret":
        return drla.decay_prefill(q, k, v, g, h0, per_channel=False, flags=flags,
                                  output_final_state=want_ht, workspace=ws)
    return drla.gdn_prefill(q, k, v, beta, g, h0, flags=flags, output_final_state=want_ht, workspace=ws)


# (kind, io, h_qk, h_v, d, lens, h0_std, want_ht)
CASES = [
    ("gdn", "bf16", 2, 4, 128, (1000,), 0.05, True),      # 4 segments, ragged tail
    ("gdn", "f16", 4, 4, 64, (777,), 0.05, True),         # 3 segments, last of 5 chunks
    ("gdn", "bf16", 4, 8, 128, (1000,), 0.0, True),       # 2 segments, 192 workgroups
    ("gdn", "bf16", 4, 16, 128, (1000,), 0.05, True),     # 16 heads: 2 paired segments, 256 workgroups
    ("ret", "f16", 4, 16, 128, (1000,), 0.05, True),      # the same, decay-only
    ("gdn", "bf16", 8, 32, 64, (900,), 0.05, True),       # 32 heads of d = 64: 2 paired segments
    ("gdn", "bf16", 4, 16, 128, (1000,), 0.05, False),    # paired, no final state
    ("gdn", "f16", 4, 12, 128, (700,), 0.05, True),       # paired, fp16, 3 value heads per key head
    ("gdn", "bf16", 2, 16, 64, (2000,), 0.05, True),      # 2 segments, 16 heads of d = 64
    ("ret", "bf16", 2, 4, 128, (600, 600), 0.05, True),   # dense batch
    ("gdn", "bf16", 2, 4, 128, (3000,), 0.05, False),     # no final state
    ("ret", "f16", 1, 4, 64, (520,), 0.0, True),          # eight chunks, the least
    ("gdn", "bf16", 1, 1, 128, (3000,), 0.05, True),      # 11 segments, last of 7 chunks
    ("gdn", "f16", 2, 2, 64, (2000,), 0.05, True),        # 8 segments
    ("ret", "bf16", 1, 1, 64, (1500,), 0.05, True),       # 6 segments, 44 workgroups
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-h{c[3]}-d{c[4]}-{c[5]}" for c in CASES])
def test_segment_split_matches_oracle_and_one_pass(drla, case, path):
    kind, io, h_qk, h_v, dk, lens, h0_std, want_ht = case
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dk, io=io,
                        g_lo=0.01, g_hi=0.2, h0_std=h0_std, seed=41)
    x = W.make_inputs(spec)
    nb = len(lens)  # a dense batch of nb equal sequences (no cu_seqlens)
    splits, wsb, rng = _splits(drla, x, path, kind, n_seqs=nb)
    print(f"case segment path={path} kind={kind} io={io} h_qk={h_qk} h_v={h_v} d={dk} lens={lens} "
          f"h0_std={h0_std} ht={want_ht} splits={splits}", flush=True)
    d = to_device(x)
    base = _base(drla, path)
    ws = _nan_workspace(wsb)
    o, ht = _call(drla, kind, d, nb, base, want_ht, ws)
    o1, ht1 = _call(drla, kind, d, nb, base | drla.SERIAL, want_ht)
    torch.cuda.synchronize()
    o, o1 = (t.reshape(-1, h_v, dk).float().cpu().numpy() for t in (o, o1))
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[io]
    eo, eo1 = rel_err(o, o_ref), rel_err(o1, o_ref)
    print(f"  rel_err o split={eo:.3e} one-pass={eo1:.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and eo <= tol and eo1 <= tol
    assert rel_err(o, o1) <= tol
    if splits:
        assert _written(ws, rng), "the split scan did not run"
    else:
        assert np.array_equal(o, o1), "a call the rule does not split differs from one pass"
    if want_ht:
        ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
        eh = rel_err(ht, ht_ref)
        print(f"  rel_err ht split={eh:.3e} one-pass={rel_err(ht1, ht_ref):.3e}", flush=True)
        assert np.isfinite(ht).all() and eh <= tol
    else:
        assert ht is None and ht1 is None


@pytest.mark.parametrize("path", PATHS)
def test_segment_split_repeatable(drla, path):
    """Two calls of the split scan on the same inputs agree bit for bit (no
    workgroup reads what another of the same call is still writing)."""
    print(f"case segment repeatable path={path}", flush=True)
    spec = W.small_spec("gdn", lens=(4000,), h_qk=2, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=42)
    d = to_device(W.make_inputs(spec))
    f = _base(drla, path)
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=f)
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=f)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_wide_call_runs_one_pass(drla):
    """Per-16-column scan: 20 heads of d = 128 need 2 x 160 paired split
    workgroups, more than a 256-CU chip holds at once: the call takes the
    one-pass scan."""
    print("case segment wide call", flush=True)
    spec = W.small_spec("gdn", lens=(1000,), h_qk=4, h_v=20, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=43)
    d = to_device(W.make_inputs(spec))
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("path", PATHS)
def test_one_packed_sequence_is_dense(drla, path):
    """One sequence passed with cu_seqlens = {0, T} takes the dense path, the
    segment split included: the same bits as the call without cu_seqlens."""
    print(f"case segment one packed sequence path={path}", flush=True)
    spec = W.small_spec("gdn", lens=(3000,), h_qk=2, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=44)
    d = to_device(W.make_inputs(spec))
    cu = torch.tensor([0, 3000], dtype=torch.int32, device="cuda")
    f = _base(drla, path)
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=f)
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], cu, cu_seqlens_host=[0, 3000],
                         flags=f)
    c = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=f | drla.SERIAL)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0]), "the split scan did not run"


# packed batches: (kind, io, h_qk, h_v, d, lens)
PACKED = [
    ("gdn", "bf16", 2, 2, 128, (1500, 700, 0, 2100)),   # 2 segments, an empty sequence
    ("gdn", "bf16", 1, 1, 128, (3000, 100, 0)),         # 5 segments; 2 chunks: segment 0 takes both
    ("ret", "f16", 1, 2, 64, (900, 2500)),              # 8 segments; 15 chunks: 1 each, segment 0 the other 8
    ("gdn", "bf16", 2, 8, 128, (1500, 2100)),           # 2 x 8 heads: 2 paired segments
    ("gdn", "bf16", 2, 4, 128, (1500, 0, 40)),          # paired; empty and one-chunk sequences
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", PACKED, ids=[f"{c[0]}-{c[1]}-h{c[3]}-d{c[4]}-{c[5]}" for c in PACKED])
def test_segment_split_packed(drla, case, path):
    """Packed input: each sequence splits its own chunks into the call's np
    segments; against the oracle and the one-pass scan."""
    kind, io, h_qk, h_v, dk, lens = case
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dk, io=io,
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=45)
    x = W.make_inputs(spec)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    splits, wsb, rng = _splits(drla, x, path, kind, n_seqs=len(lens), cu_host=cu_host)
    print(f"case segment packed path={path} kind={kind} io={io} h_qk={h_qk} h_v={h_v} d={dk} "
          f"lens={lens} splits={splits}", flush=True)
    d = to_device(x)
    base = _base(drla, path)
    ws = _nan_workspace(wsb)

    def call(flags, ws=None):
        if kind == "ret":
            return drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                                      cu_seqlens_host=d["cu_host"], per_channel=False, flags=flags,
                                      workspace=ws)
        return drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                                cu_seqlens_host=d["cu_host"], flags=flags, workspace=ws)
    o, ht = call(base, ws)
    o1, ht1 = call(base | drla.SERIAL)
    torch.cuda.synchronize()
    o, o1 = o.float().cpu().numpy(), o1.float().cpu().numpy()
    ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[io]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} one-pass o={rel_err(o1, o_ref):.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    assert eo <= tol and eh <= tol
    assert rel_err(o, o1) <= tol and rel_err(ht, ht1) <= tol
    if splits:
        assert _written(ws, rng), "the split scan did not run"
    else:
        assert np.array_equal(o, o1)
