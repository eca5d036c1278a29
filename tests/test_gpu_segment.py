"""The segment-split scan of dense calls that leave most of the chip idle.

Such a call splits every sequence's chunks into np segments (np = 2 when
three scan workgroups per column block fill a third of the chip, up to 16
for a single head).  Segment 0 is scanned from the initial state; every
later one twice at the same time: from a zero state with the real values,
and from the identity with V = 0 (the linear map of the entering state on
the outputs and on the final state).  A compose kernel chains the entering
states and a fix-up adds each segment's map applied to its entering state.
The cases take 2, 3, 4, 6, 8 and 11 segments, an uneven last segment,
workgroup counts that are not a multiple of 8, ragged last chunks, grouped
heads, dk = 64 and 128, a dense batch, no initial state, no final state, the
fewest chunks a split takes, and the decay-only form; each is checked
against the oracle, and against the one-pass scan of the same call
(DRLA_SERIAL), which must differ in rounding somewhere (else the split did
not run).  A call too wide for the split equals the one-pass scan bit for
bit."""
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


def _call(drla, kind, d, dense_batch, flags, want_ht):
    q, k, v, beta, g, h0 = d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"]
    if dense_batch > 1:
        q, k, v = (x.view(dense_batch, -1, *x.shape[1:]) for x in (q, k, v))
        beta, g = (x.view(dense_batch, -1, *x.shape[1:]) for x in (beta, g))
    if kind == "ret":
        return drla.decay_prefill(q, k, v, g, h0, per_channel=False, flags=flags,
                                  output_final_state=want_ht)
    return drla.gdn_prefill(q, k, v, beta, g, h0, flags=flags, output_final_state=want_ht)


# (kind, io, h_qk, h_v, d, lens, h0_std, want_ht)
CASES = [
    ("gdn", "bf16", 2, 4, 128, (1000,), 0.05, True),      # 4 segments, ragged tail
    ("gdn", "f16", 4, 4, 64, (777,), 0.05, True),         # 3 segments, last of 5 chunks
    ("gdn", "bf16", 4, 8, 128, (1000,), 0.0, True),       # 2 segments, 192 workgroups
    ("gdn", "bf16", 2, 16, 64, (2000,), 0.05, True),      # 2 segments, 16 heads of d = 64
    ("ret", "bf16", 2, 4, 128, (600, 600), 0.05, True),   # dense batch
    ("gdn", "bf16", 2, 4, 128, (3000,), 0.05, False),     # no final state
    ("ret", "f16", 1, 4, 64, (520,), 0.0, True),          # eight chunks, the least
    ("gdn", "bf16", 1, 1, 128, (3000,), 0.05, True),      # 11 segments, last of 7 chunks
    ("gdn", "f16", 2, 2, 64, (2000,), 0.05, True),        # 8 segments
    ("ret", "bf16", 1, 1, 64, (1500,), 0.05, True),       # 6 segments, 44 workgroups
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-h{c[3]}-d{c[4]}-{c[5]}" for c in CASES])
def test_segment_split_matches_oracle_and_one_pass(drla, case):
    kind, io, h_qk, h_v, dk, lens, h0_std, want_ht = case
    print(f"case segment kind={kind} io={io} h_qk={h_qk} h_v={h_v} d={dk} lens={lens} "
          f"h0_std={h0_std} ht={want_ht}", flush=True)
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dk, io=io,
                        g_lo=0.01, g_hi=0.2, h0_std=h0_std, seed=41)
    x = W.make_inputs(spec)
    d = to_device(x)
    nb = len(lens)
    o, ht = _call(drla, kind, d, nb, 0, want_ht)
    o1, ht1 = _call(drla, kind, d, nb, drla.SERIAL, want_ht)
    torch.cuda.synchronize()
    o, o1 = (t.reshape(-1, h_v, dk).float().cpu().numpy() for t in (o, o1))
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[io]
    eo, eo1 = rel_err(o, o_ref), rel_err(o1, o_ref)
    print(f"  rel_err o split={eo:.3e} one-pass={eo1:.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and eo <= tol
    assert rel_err(o, o1) <= tol
    assert not np.array_equal(o, o1), "the split scan did not run"
    if want_ht:
        ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
        eh = rel_err(ht, ht_ref)
        print(f"  rel_err ht split={eh:.3e} one-pass={rel_err(ht1, ht_ref):.3e}", flush=True)
        assert np.isfinite(ht).all() and eh <= tol
    else:
        assert ht is None and ht1 is None


def test_segment_split_repeatable(drla):
    """Two calls of the split scan on the same inputs agree bit for bit (no
    workgroup reads what another of the same call is still writing)."""
    print("case segment repeatable", flush=True)
    spec = W.small_spec("gdn", lens=(4000,), h_qk=2, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=42)
    d = to_device(W.make_inputs(spec))
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_wide_call_runs_one_pass(drla):
    """16 heads of d = 128 need 384 split workgroups, more than a 256-CU chip
    holds at once: the call takes the one-pass scan."""
    print("case segment wide call", flush=True)
    spec = W.small_spec("gdn", lens=(1000,), h_qk=4, h_v=16, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=43)
    d = to_device(W.make_inputs(spec))
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_one_packed_sequence_is_dense(drla):
    """One sequence passed with cu_seqlens = {0, T} takes the dense path, the
    segment split included: the same bits as the call without cu_seqlens."""
    print("case segment one packed sequence", flush=True)
    spec = W.small_spec("gdn", lens=(3000,), h_qk=2, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=44)
    d = to_device(W.make_inputs(spec))
    cu = torch.tensor([0, 3000], dtype=torch.int32, device="cuda")
    a = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    b = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], cu, cu_seqlens_host=[0, 3000])
    c = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0]), "the split scan did not run"


# packed batches: (kind, io, h_qk, h_v, d, lens)
PACKED = [
    ("gdn", "bf16", 2, 2, 128, (1500, 700, 0, 2100)),   # 2 segments, an empty sequence
    ("gdn", "bf16", 1, 1, 128, (3000, 100, 0)),         # 5 segments; 2 chunks: the last takes both
    ("ret", "f16", 1, 2, 64, (900, 2500)),              # 8 segments, one of 1 chunk each but the last
]


@pytest.mark.parametrize("case", PACKED, ids=[f"{c[0]}-{c[1]}-h{c[3]}-d{c[4]}-{c[5]}" for c in PACKED])
def test_segment_split_packed(drla, case):
    """Packed input: each sequence splits its own chunks into the call's np
    segments; against the oracle and the one-pass scan."""
    kind, io, h_qk, h_v, dk, lens = case
    print(f"case segment packed kind={kind} io={io} h_qk={h_qk} h_v={h_v} d={dk} lens={lens}", flush=True)
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dk, io=io,
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=45)
    x = W.make_inputs(spec)
    d = to_device(x)

    def call(flags):
        if kind == "ret":
            return drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                                      cu_seqlens_host=d["cu_host"], per_channel=False, flags=flags)
        return drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                                cu_seqlens_host=d["cu_host"], flags=flags)
    o, ht = call(0)
    o1, ht1 = call(drla.SERIAL)
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
    assert not np.array_equal(o, o1), "the split scan did not run"
