"""The head-resident scan (DRLA_HEAD_SCAN) against the fp64 oracle: one
workgroup per (sequence, head) unit holding all dv state columns, with the
segment split when the units leave compute units idle.  Shapes the segment
tests do not take: dk != dv (one pass), packed ragged batches with grouped
heads and empty or one-token sequences, fp16, the decay-only form, and the
H16 d128 T4096 workload at full size.  Bar as the other parity tests."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, nmse, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _run(drla, x, flags):
    d = to_device(x)
    if x["kind"] == "ret":
        o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                                   cu_seqlens_host=d["cu_host"], per_channel=False, flags=flags)
    else:
        o, ht = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                                 cu_seqlens_host=d["cu_host"], flags=flags)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ht.cpu().numpy()


def _check(tag, x, o, ht):
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[x["io"]]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"{tag}: rel_err o={eo:.3e} ht={eh:.3e} nmse o={nmse(o, o_ref):.2e} (tol {tol:g})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    assert eo <= tol and eh <= tol
    return o_ref, ht_ref


# (kind, io, h_qk, h_v, dk, dv, lens, h0_std)
CASES = [
    ("gdn", "bf16", 2, 2, 64, 128, (300,), 0.05),                       # dk != dv: one pass
    ("gdn", "bf16", 2, 4, 128, 64, (1, 63, 64, 65, 130, 0, 7), 0.05),   # dk != dv, packed ragged
    ("gdn", "bf16", 2, 4, 128, 128, (1, 63, 64, 65, 130, 0, 7), 0.05),  # packed ragged, grouped
    ("gdn", "f16", 1, 3, 128, 128, (64, 700, 5, 300, 0, 129), 0.05),    # unsorted lengths
    ("ret", "bf16", 2, 2, 64, 64, (200, 333), 0.0),                     # decay-only, packed
    ("gdn", "bf16", 1, 1, 64, 64, (5000,), 0.05),                       # one unit, many segments
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[4]}x{c[5]}-h{c[3]}-{len(c[6])}seq" for c in CASES])
def test_head_scan_matches_oracle(drla, case):
    kind, io, h_qk, h_v, dk, dv, lens, h0_std = case
    print(f"case head-scan kind={kind} io={io} h_qk={h_qk} h_v={h_v} dk={dk} dv={dv} lens={lens}", flush=True)
    spec = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv, io=io,
                        g_lo=0.01, g_hi=0.2, h0_std=h0_std, seed=51)
    x = W.make_inputs(spec)
    o, ht = _run(drla, x, drla.HEAD_SCAN)
    _check(f"head-scan {kind}/{io}/{dk}x{dv}", x, o, ht)
    if h0_std > 0 and x["varlen"]:
        # an empty sequence returns its initial state unchanged
        for s, L in enumerate(lens):
            if L == 0:
                np.testing.assert_array_equal(ht[s], x["h0"][s])


def test_head_scan_workload_gdn_prefill(drla):
    """H16 d128 T4096 (16 units x 16 segments of 4 chunks) against the oracle,
    and against the default scan of the same call."""
    spec = W.spec_by_name("gdn_prefill")
    print("case head-scan workload gdn_prefill", flush=True)
    x = W.make_inputs(spec)
    o, ht = _run(drla, x, drla.HEAD_SCAN)
    o_ref, ht_ref = _check("head-scan gdn_prefill", x, o, ht)
    o1, ht1 = _run(drla, x, 0)
    assert rel_err(o, o1) <= TOL["bf16"] and rel_err(ht, ht1) <= TOL["bf16"]


def test_head_scan_repeatable(drla):
    """Two split calls on the same inputs agree bit for bit."""
    spec = W.small_spec("gdn", lens=(4000,), h_qk=2, h_v=2, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=52)
    x = W.make_inputs(spec)
    a = _run(drla, x, drla.HEAD_SCAN)
    b = _run(drla, x, drla.HEAD_SCAN)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("h_v,T,io", [(16, 16384, "bf16"), (8, 16384, "f16")])
def test_automatic_head_scan(drla, h_v, T, io):
    """Without flags the call takes the head-resident scan at these shapes
    (its timing model predicts it faster; the layout shows the hs region):
    against the oracle and against the per-16-column scan (DRLA_SERIAL)."""
    print(f"case automatic head scan h_v={h_v} T={T} io={io}", flush=True)
    # weak gates, so that the state entering each segment still matters
    spec = W.small_spec("gdn", lens=(T,), h_qk=h_v // 2, h_v=h_v, dk=128, dv=128, io=io,
                        g_lo=0.001, g_hi=0.05, h0_std=0.05, seed=61)
    x = W.make_inputs(spec)
    d = to_device(x)
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype)
    assert lay["hs"] > 0 and lay["seg"] == 0, "the layout should show the head-resident scan"
    ws = torch.full((lay["total"],), 255, dtype=torch.uint8, device="cuda")
    o, ht = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], workspace=ws)
    torch.cuda.synchronize()
    first_set = ws[lay["hs"]:lay["hs"] + h_v * 128 * 128 * 4].view(torch.float32)
    assert bool(torch.isfinite(first_set).all()), "the head-resident split did not run"
    o1, ht1 = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    o, o1 = o.float().cpu().numpy(), o1.float().cpu().numpy()
    ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    tol = TOL[io]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (column scan {rel_err(o1, o_ref):.3e})", flush=True)
    assert np.isfinite(o).all() and eo <= tol and eh <= tol
    assert rel_err(o1, o_ref) <= tol and rel_err(o, o1) <= tol


def test_automatic_head_scan_many_units(drla):
    """A packed batch with more (sequence, head, 16-column) chains than the
    chip has compute units (64 sequences of 512 tokens, 8 heads: 4,096
    chains) takes the head-resident scan in one pass without flags (the
    layout records the choice): against the oracle and against the
    per-16-column scan (DRLA_SERIAL)."""
    lens = (512,) * 64
    print(f"case automatic head scan, packed {len(lens)} x {lens[0]}, h_v=8", flush=True)
    spec = W.small_spec("gdn", lens=lens, h_qk=4, h_v=8, dk=128, dv=128, io="bf16",
                        g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=62, varlen=True)
    x = W.make_inputs(spec)
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, cu_seqlens_host=cu_host)
    assert lay["head_scan"] == 1 and lay["seg"] == 0 and lay["hs"] == 0
    ws = torch.full((lay["total"],), 255, dtype=torch.uint8, device="cuda")
    o, ht = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                             cu_seqlens_host=cu_host, workspace=ws)
    o1, ht1 = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                               cu_seqlens_host=cu_host, flags=drla.SERIAL)
    torch.cuda.synchronize()
    o, o1 = o.float().cpu().numpy(), o1.float().cpu().numpy()
    ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (column scan {rel_err(o1, o_ref):.3e})", flush=True)
    assert np.isfinite(o).all() and eo <= TOL["bf16"] and eh <= TOL["bf16"]
    assert rel_err(o1, o_ref) <= TOL["bf16"] and rel_err(ht1, ht_ref) <= TOL["bf16"]


def test_column_scan_flag(drla):
    """DRLA_COLUMN_SCAN at a shape where the model takes the head-resident
    scan (8 heads, 16,384 tokens): the layout shows the per-16-column scan's
    segment region, the workspace region holding the segments' states is
    written, and o and ht match the oracle and the one-pass scan."""
    print("case column-scan flag h_v=8 T=16384", flush=True)
    spec = W.small_spec("gdn", lens=(16384,), h_qk=4, h_v=8, dk=128, dv=128, io="bf16",
                        g_lo=0.001, g_hi=0.05, h0_std=0.05, seed=63)
    x = W.make_inputs(spec)
    d = to_device(x)
    assert drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype)["head_scan"] == 1
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, flags=drla.COLUMN_SCAN)
    assert lay["head_scan"] == 0 and lay["hs"] == 0 and lay["seg"] > 0
    ws = torch.full((lay["total"],), 255, dtype=torch.uint8, device="cuda")
    o, ht = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], workspace=ws,
                             flags=drla.COLUMN_SCAN)
    torch.cuda.synchronize()
    mid = ws[lay["seg"]:lay["seg"] + 8 * 128 * 128 * 4].view(torch.float32)
    assert bool(torch.isfinite(mid).all()), "the per-16-column split did not run"
    o1, ht1 = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    o, o1 = o.float().cpu().numpy(), o1.float().cpu().numpy()
    ht, ht1 = ht.cpu().numpy(), ht1.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e}", flush=True)
    assert np.isfinite(o).all() and eo <= TOL["bf16"] and eh <= TOL["bf16"]
    assert rel_err(o, o1) <= TOL["bf16"] and rel_err(ht, ht1) <= TOL["bf16"]
    with pytest.raises(RuntimeError):
        drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"],
                         flags=drla.COLUMN_SCAN | drla.HEAD_SCAN)
