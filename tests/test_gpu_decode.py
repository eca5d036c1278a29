"""Parity of the decode step (gdn_decode / kda_decode, through the C ABI)
with the fp64 oracle's token recurrence.

Same bar as prefill: max|x - y| / max|y| <= 2e-2 for bf16 inputs, 5e-3 for
fp16 and 1e-4 for fp32, on o and on the state."""
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


def _inputs(kind, io, dk, dv, lens, h_qk=2, h_v=4, h0_std=0.05, seed=5):
    g_lo, g_hi = (0.01, 0.2) if kind == "gdn" else (0.005, 0.15)
    s = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv, io=io, g_lo=g_lo,
                     g_hi=g_hi, h0_std=h0_std, seed=seed, varlen=True)
    return W.make_inputs(s)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("io", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_step_matches_oracle(drla, kind, io, dk, dv):
    """Six sequences, one token each, grouped heads, a nonzero state."""
    print(f"case decode kind={kind} io={io} dk={dk} dv={dv}", flush=True)
    x = _inputs(kind, io, dk, dv, lens=(1,) * 6)
    d = to_device(x)
    fn = drla.kda_decode if kind == "kda" else drla.gdn_decode
    o, ht = fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = run_oracle(x)
    _check(f"decode {kind}/{io}/{dk}x{dv}", io, _np(o), _np(ht), o_ref, ht_ref)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_decode_steps_continue_a_sequence(drla, kind):
    """Five decode steps in place on three sequences equal the oracle on
    the three five-token sequences, output by output."""
    print(f"case decode-steps kind={kind}", flush=True)
    T, N = 5, 3
    x = _inputs(kind, "bf16", 128, 128, lens=(T,) * N, h_qk=1, h_v=2)
    d = to_device(x)
    fn = drla.kda_decode if kind == "kda" else drla.gdn_decode
    state = d["h0"].clone()
    outs = []
    for t in range(T):
        rows = [n * T + t for n in range(N)]
        pick = lambda a: a[rows].contiguous()
        o, ht = fn(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d["beta"]), pick(d["g"]),
                   state, in_place=True)
        assert ht.data_ptr() == state.data_ptr()
        outs.append(o.clone())
    torch.cuda.synchronize()
    o_all = torch.stack(outs, dim=1).reshape(N * T, 2, 128)   # sequence-major, as packed
    o_ref, ht_ref = run_oracle(x)
    _check(f"decode-steps {kind}", "bf16", _np(o_all), _np(state), o_ref, ht_ref)


def test_decode_without_state_starts_from_zero(drla):
    x = _inputs("gdn", "f32", 64, 64, lens=(1,) * 4, h0_std=0.0)
    d = to_device(x)
    o1, h1 = drla.gdn_decode(d["q"], d["k"], d["v"], d["beta"], d["g"], None)
    z = torch.zeros_like(h1)
    o2, h2 = drla.gdn_decode(d["q"], d["k"], d["v"], d["beta"], d["g"], z)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, ht_ref = run_oracle(x)
    _check("decode zero state", "f32", _np(o1), _np(h1), o_ref, ht_ref)


def test_decode_matches_prefill_of_one_token(drla):
    """The decode kernel and the chunked prefill (one-token sequences) agree."""
    x = _inputs("kda", "bf16", 128, 128, lens=(1,) * 8)
    d = to_device(x)
    o1, h1 = drla.kda_decode(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])
    o2, h2 = drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                              cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    assert rel_err(_np(o1), _np(o2)) <= TOL["bf16"] and rel_err(_np(h1), _np(h2)) <= TOL["bf16"]
