"""Guard bands around every buffer a prefill call writes (GPU).

The workspace, the output o and the final state are carved out of larger
allocations whose every byte is 0xFF (a NaN in any float type); 64 KiB on
either side of each is a guard band.  After the call the bands must still
hold 0xFF byte for byte (no write outside the buffer the caller passed),
and the results must be finite and match the oracle: the workspace starts
as NaN, so a read of any workspace byte the call did not write first would
reach the result.  Cases: GDN and KDA in bf16, fp16 and fp32, packed ragged
sequences with grouped heads, the per-16-column scan (default), its
segment split, the head-resident scan and the one-pass scan, decay-only."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, nmse, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 64 << 10


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _guarded(nbytes):
    """(allocation, view of nbytes inside it) with GUARD bytes of 0xFF on
    both sides."""
    buf = torch.full((nbytes + 2 * GUARD,), 255, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + nbytes]


def _bands_intact(buf, nbytes):
    lo, hi = buf[:GUARD], buf[GUARD + nbytes:]
    return bool((lo == 255).all()) and bool((hi == 255).all())


CASES = [
    # kind, io, lens, h_qk, h_v, dk, dv, flag name
    ("gdn", "bf16", (200, 1, 0, 130), 1, 2, 128, 128, "default"),
    ("gdn", "bf16", (4096,), 2, 2, 128, 128, "default"),        # segment split
    ("gdn", "bf16", (4096,), 2, 2, 128, 128, "HEAD_SCAN"),
    ("gdn", "bf16", (700, 65), 1, 3, 128, 128, "SERIAL"),
    ("gdn", "f16", (129, 63), 2, 4, 64, 128, "default"),
    ("gdn", "f32", (200, 7), 1, 2, 128, 64, "default"),
    ("kda", "bf16", (200, 1, 0, 130), 1, 2, 128, 128, "default"),
    ("kda", "f16", (300,), 2, 2, 64, 64, "default"),
    ("kda", "f32", (130, 64), 1, 2, 128, 128, "default"),
    ("gla", "bf16", (257, 3), 1, 2, 128, 128, "default"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[7]}-{'x'.join(map(str, c[2]))}")
def test_writes_stay_inside_buffers(drla, case):
    kind, io, lens, h_qk, h_v, dk, dv, flag = case
    print(f"case guard {case}", flush=True)
    x = W.make_inputs(W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv, io=io,
                                   g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=17,
                                   varlen=len(lens) > 1))
    d = to_device(x)
    tdt = d["q"].dtype
    flags = getattr(drla, flag) if flag != "default" else 0
    if kind == "gla":
        flags |= drla.DECAY_ONLY
    cu_host = [int(c) for c in x["cu_seqlens"]] if x["varlen"] else None
    n = len(lens) if x["varlen"] else 1
    T = int(x["cu_seqlens"][-1])
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, tdt, n_seqs=n, cu_seqlens_host=cu_host,
                                kda=kind in ("kda", "gla"), flags=flags)
    need = int(lay["total"])
    wbuf, ws = _guarded(need)
    es = d["q"].element_size()
    obuf, ob = _guarded(T * h_v * dv * es)
    hbuf, hb = _guarded(n * h_v * dk * dv * 4)
    o = ob.view(tdt).view(T, h_v, dv)
    ht = hb.view(torch.float32).view(n, h_v, dk, dv)
    fn = drla.kda_prefill if kind in ("kda", "gla") else drla.gdn_prefill
    beta = None if kind == "gla" else d["beta"]
    fn(d["q"], d["k"], d["v"], beta, d["g"], d["h0"], d["cu"], cu_seqlens_host=cu_host,
       workspace=ws, out=o, final_state=ht, flags=flags)
    torch.cuda.synchronize()
    assert _bands_intact(wbuf, need), "write outside the workspace"
    assert _bands_intact(obuf, ob.numel()), "write outside o"
    assert _bands_intact(hbuf, hb.numel()), "write outside the final state"
    on, hn = o.float().cpu().numpy(), ht.cpu().numpy()
    assert np.isfinite(on).all() and np.isfinite(hn).all(), "a NaN workspace byte reached the result"
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(on, o_ref), rel_err(hn, ht_ref)
    print(f"guard {kind}/{io}/{flag}: rel_err o={eo:.3e} ht={eh:.3e} nmse o={nmse(on, o_ref):.2e}",
          flush=True)
    assert eo <= TOL[io] and eh <= TOL[io]
