"""Seeded random configurations through the C ABI against the fp64 oracle.

Each case draws, from its own seed: the gate kind (GDN, KDA, and the
decay-only forms with a scalar or per-channel gate), the io dtype, dk and
dv, the head grouping, one dense sequence or a packed batch with ragged
(sometimes empty) sequences, a zero or random initial state, and the gate
strength up to the range the ABI documents for that kind and dtype.  Bar:
the same per-dtype bound as the other parity tests."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# log-gate bounds -U(lo, hi) over the range the ABI documents: any for a
# scalar gate; per-channel gates |g| < 11 per token (drawn up to 8)
_G_HI = {("scalar", "bf16"): 8.0, ("scalar", "f16"): 8.0, ("scalar", "f32"): 8.0,
         ("channel", "bf16"): 8.0, ("channel", "f32"): 8.0, ("channel", "f16"): 8.0}


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    kind = ["gdn", "kda", "ret", "gla"][int(rng.integers(0, 4))]
    io = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
    dk, dv = (int(x) for x in rng.choice([64, 128], size=2))
    h_qk = int(rng.integers(1, 3))
    h_v = h_qk * int(rng.choice([1, 2, 4]))
    if rng.random() < 0.3:
        lens = (int(rng.integers(1, 700)),)
    else:
        n = int(rng.integers(2, 6))
        lens = tuple(int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 400, size=n))
    gate = "scalar" if kind in ("gdn", "ret") else "channel"
    hi = float(rng.uniform(0.02, 1.0)) * _G_HI[(gate, io)]
    lo = float(rng.uniform(0.0, 0.5)) * hi
    h0_std = float(rng.choice([0.0, 0.05]))
    spec = W.Spec(f"random{seed}", kind, lens, h_qk, h_v, dk, dv, io, lo, hi, h0_std,
                  varlen=len(lens) > 1, seed=seed)
    return spec


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("seed", range(24))
def test_random_configuration(drla, seed):
    spec = _draw(seed)
    print(f"case random seed={seed}: kind={spec.kind} io={spec.io} dk={spec.dk} dv={spec.dv} "
          f"h_qk={spec.h_qk} h_v={spec.h_v} lens={spec.lens} g=-U({spec.g_lo:.3f},{spec.g_hi:.3f}) "
          f"h0_std={spec.h0_std}", flush=True)
    x = W.make_inputs(spec)
    d = to_device(x)
    if spec.kind in ("ret", "gla"):
        o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                                   cu_seqlens_host=d["cu_host"], per_channel=spec.kind == "gla")
    else:
        fn = drla.kda_prefill if spec.kind == "kda" else drla.gdn_prefill
        o, ht = fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                   cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    tol = TOL[spec.io]
    eo = 0.0 if o.size == 0 else rel_err(o, o_ref) if np.abs(o_ref).max() > 0 else float(np.abs(o).max())
    eh = rel_err(ht, ht_ref) if np.abs(ht_ref).max() > 0 else float(np.abs(ht).max())
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eh <= tol


def _draw_paired(seed):
    """A scalar-gate 16-bit call whose (sequence, head, 16-column) chains
    number 86 to 128: too many for three workgroups each on 256 compute
    units, so the scan splits every sequence into two segments with paired
    chains (segment 0 longer than segment 1)."""
    rng = np.random.default_rng(2000 + seed)
    kind = ["gdn", "ret"][int(rng.integers(0, 2))]
    io = ["bf16", "f16"][int(rng.integers(0, 2))]
    d = int(rng.choice([64, 128]))
    lo_u, hi_u = (11, 16) if d == 128 else (22, 32)
    while True:
        n = int(rng.integers(1, 4))
        h_qk = int(rng.choice([1, 2, 4]))
        h_v = h_qk * int(rng.choice([1, 2, 4, 8]))
        if lo_u <= n * h_v <= hi_u:
            break
    longest = int(rng.integers(460, 1400))
    lens = [longest] + [int(x) if rng.random() > 0.2 else 0 for x in rng.integers(1, 1400, size=n - 1)]
    rng.shuffle(lens)
    hi = float(rng.uniform(0.02, 1.0)) * 8.0
    lo = float(rng.uniform(0.0, 0.5)) * hi
    h0_std = float(rng.choice([0.0, 0.05]))
    return W.Spec(f"paired{seed}", kind, tuple(lens), h_qk, h_v, d, d, io, lo, hi, h0_std,
                  varlen=n > 1, seed=seed)


@pytest.mark.parametrize("seed", range(8))
def test_random_paired_split(drla, seed):
    spec = _draw_paired(seed)
    print(f"case random paired seed={seed}: kind={spec.kind} io={spec.io} d={spec.dk} h_qk={spec.h_qk} "
          f"h_v={spec.h_v} lens={spec.lens} g=-U({spec.g_lo:.3f},{spec.g_hi:.3f}) h0_std={spec.h0_std}",
          flush=True)
    x = W.make_inputs(spec)
    d = to_device(x)
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, n_seqs=len(spec.lens),
                                cu_seqlens_host=d["cu_host"], kda=False,
                                flags=drla.DECAY_ONLY if spec.kind == "ret" else 0)
    assert lay["seg"] > 0, "the call should take the segment split"
    if spec.kind == "ret":
        o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], d["cu"],
                                   cu_seqlens_host=d["cu_host"], per_channel=False)
    else:
        o, ht = drla.gdn_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                                 cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    o_ref, ht_ref = run_oracle(x)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    tol = TOL[spec.io]
    eo = rel_err(o, o_ref) if np.abs(o_ref).max() > 0 else float(np.abs(o).max())
    eh = rel_err(ht, ht_ref) if np.abs(ht_ref).max() > 0 else float(np.abs(ht).max())
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eh <= tol
