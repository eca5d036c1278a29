"""Parity of decay-only linear attention (decay_prefill / decay_decode, the
RetNet / GLA form without the delta rule; through the C ABI) with the fp64
oracle's decay-only recurrence.  Bars as for the delta rule: 2e-2 (bf16),
5e-3 (fp16), 1e-4 (fp32) on o and on the final state."""
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


def _np(t):
    return t.float().cpu().numpy()


def _check(tag, io, o, ht, o_ref, ht_ref):
    tol = TOL[io]
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"{tag}: rel_err o={eo:.3e} ht={eh:.3e} nmse o={nmse(o, o_ref):.2e} (tol {tol:g})",
          flush=True)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    assert eo <= tol and eh <= tol, tag


def _inputs(kind, io, dk, dv, lens, h_qk=1, h_v=2, h0_std=0.05, seed=9, g_lo=0.01, g_hi=0.2,
            varlen=True):
    s = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv, io=io, g_lo=g_lo,
                     g_hi=g_hi, h0_std=h0_std, seed=seed, varlen=varlen)
    return W.make_inputs(s)


@pytest.mark.parametrize("kind", ["ret", "gla"])
@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_decay_prefill_matches_oracle(drla, kind, io, dk, dv):
    """Packed ragged sequences (several chunks, a one-token sequence, a
    short tail), grouped heads, a nonzero initial state."""
    print(f"case decay kind={kind} io={io} dk={dk} dv={dv}", flush=True)
    x = _inputs(kind, io, dk, dv, lens=(200, 1, 63, 130))
    d = to_device(x)
    o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                               cu_seqlens_host=d["cu_host"], per_channel=kind == "gla")
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(x)
    _check(f"decay {kind}/{io}/{dk}x{dv}", io, _np(o), _np(ht), o_ref, ht_ref)


@pytest.mark.parametrize("kind", ["ret", "gla"])
def test_decay_prefill_fast_forgetting(drla, kind):
    """Strong gates (up to e^-1 per token): the in-chunk decay factors span
    e^-64, far below any state magnitude."""
    x = _inputs(kind, "bf16", 128, 128, lens=(300,), g_lo=0.2, g_hi=1.0, varlen=False)
    d = to_device(x)
    o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"],
                               per_channel=kind == "gla")
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(x)
    _check(f"decay fast {kind}", "bf16", _np(o), _np(ht), o_ref, ht_ref)


@pytest.mark.parametrize("kind", ["ret", "gla"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decay_decode_matches_oracle(drla, kind, io):
    x = _inputs(kind, io, 128, 128, lens=(1,) * 6, h_qk=2, h_v=4)
    d = to_device(x)
    o, ht = drla.decay_decode(d["q"], d["k"], d["v"], d["g"], d["h0"], per_channel=kind == "gla")
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(x)
    _check(f"decay decode {kind}/{io}", io, _np(o), _np(ht), o_ref, ht_ref)
