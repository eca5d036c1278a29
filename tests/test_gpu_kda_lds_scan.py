"""KDA calls with 16-bit inputs whose prep operands (K e^B, K~^T and Q e^B,
3 x 64 x dk elements per head and chunk) reach 112 MiB take the LDS-fed scan
(the launcher's rule; smaller ones take the register-fed scan, which the
other KDA tests cover).  Here: the whole call against the fp64 oracle in one
pass and with the segment split, V' and the per-chunk states of one head
against the chunkwise oracle's intermediates, and decay-only attention with
the per-channel gate.  Bar as the other parity tests."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, decode_blocks, kmap_contiguous, nmse, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LDS_SCAN_BYTES = 112 << 20


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _operand_bytes(T, h_v, dk):
    return -(-T // 64) * h_v * 3 * 64 * dk * 2


def _inputs(T, h_qk, h_v, io, seed, dk=128, dv=128):
    spec = W.small_spec("kda", lens=(T,), h_qk=h_qk, h_v=h_v, dk=dk, dv=dv, io=io,
                        g_lo=0.005, g_hi=0.15, h0_std=0.02, seed=seed)
    return W.make_inputs(spec)


@pytest.mark.parametrize("T,h_qk,h_v,io,serial", [
    (16384, 8, 16, "bf16", True),    # one pass, two value heads per query/key head
    (32768, 8, 8, "f16", True),
    (65536, 8, 8, "bf16", False),    # 64 column chains: the two-segment split
])
def test_kda_lds_scan_matches_oracle(drla, T, h_qk, h_v, io, serial):
    assert _operand_bytes(T, h_v, 128) >= LDS_SCAN_BYTES
    print(f"case kda lds scan T={T} h_qk={h_qk} h_v={h_v} io={io} serial={serial}", flush=True)
    x = _inputs(T, h_qk, h_v, io, seed=71)
    d = to_device(x)
    flags = drla.SERIAL if serial else 0
    if not serial:
        lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, kda=True)
        assert lay["seg"] > 0, "the call should take the segment split"
    o, ht = drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=flags)
    torch.cuda.synchronize()
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    del d
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} nmse o={nmse(o, o_ref):.2e} (tol {TOL[io]:g})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    assert eo <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("T,dk,dv", [(32768, 64, 64), (16384, 128, 64), (32768, 64, 128)])
def test_kda_lds_scan_other_head_dims(drla, T, dk, dv):
    """The other (dk, dv) the scan serves, at 192 MiB of prep operands (16
    heads, one pass)."""
    assert _operand_bytes(T, 16, dk) >= LDS_SCAN_BYTES
    print(f"case kda lds scan T={T} dk={dk} dv={dv}", flush=True)
    x = _inputs(T, 16, 16, "bf16", seed=74, dk=dk, dv=dv)
    d = to_device(x)
    o, ht = drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], flags=drla.SERIAL)
    torch.cuda.synchronize()
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    del d
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (tol {TOL['bf16']:g})", flush=True)
    assert np.isfinite(o).all() and eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_kda_lds_scan_intermediates(drla):
    """V' and the state entering every chunk of value head 5, as the LDS-fed
    KDA scan stores them with DRLA_KEEP_INTERMEDIATES, against the chunkwise
    oracle's on that head alone."""
    import oracle
    T, h_qk, h_v, dk, dv, h = 16384, 8, 16, 128, 128, 5
    assert _operand_bytes(T, h_v, dk) >= LDS_SCAN_BYTES
    print(f"case kda lds scan intermediates T={T} h_v={h_v} head={h}", flush=True)
    x = _inputs(T, h_qk, h_v, "bf16", seed=72)
    d = to_device(x)
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, kda=True,
                                flags=drla.KEEP_INTERMEDIATES)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    drla.kda_prefill(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], workspace=ws,
                     flags=drla.KEEP_INTERMEDIATES)
    torch.cuda.synchronize()
    nc = lay["n_chunks"]

    def head_region(off, per):
        # every chunk of head h: (h nc + c) per elements of two bytes each
        a = off + h * nc * per * 2
        return ws[a:a + nc * per * 2].view(torch.bfloat16).float().cpu().numpy()
    vp = head_region(lay["vp"], 64 * dv)
    hs = head_region(lay["h"], dk * dv)
    del ws, d
    hk = h // (h_v // h_qk)
    _, _, inter = oracle.chunked(x["q"][:, hk:hk + 1], x["k"][:, hk:hk + 1], x["v"][:, h:h + 1],
                                 x["beta"][:, h:h + 1], x["g"][:, h:h + 1], x["h0"][:, h:h + 1],
                                 kda=True, intermediates=True)
    worst = {"V'": 0.0, "h": 0.0}
    for c in range(nc):
        it = inter[0][c]
        n = it["W"].shape[0]
        got_vp = decode_blocks(vp[c * 64 * dv:(c + 1) * 64 * dv], dv, 64, "outer_major").T[:n]
        got_h = decode_blocks(hs[c * dk * dv:(c + 1) * dk * dv], dv, dk, "outer_major", kmap_contiguous).T
        worst["V'"] = max(worst["V'"], rel_err(got_vp, it["Vp"]))
        worst["h"] = max(worst["h"], rel_err(got_h, it["h"]))
    print("  worst", {k: f"{v:.2e}" for k, v in worst.items()}, flush=True)
    for name, e in worst.items():
        assert e <= TOL["bf16"], f"{name}: {e}"


def test_gla_lds_scan_matches_oracle(drla):
    """Decay-only linear attention with the per-channel gate (decay_prefill,
    per_channel) at the same size takes the same scan (R = V, no X term)."""
    T, h_qk, h_v = 16384, 16, 16
    assert _operand_bytes(T, h_v, 128) >= LDS_SCAN_BYTES
    print(f"case gla lds scan T={T} h_v={h_v}", flush=True)
    spec = W.small_spec("gla", lens=(T,), h_qk=h_qk, h_v=h_v, dk=128, dv=128, io="bf16",
                        g_lo=0.005, g_hi=0.15, h0_std=0.02, seed=73)
    x = W.make_inputs(spec)
    d = to_device(x)
    o, ht = drla.decay_prefill(d["q"], d["k"], d["v"], d["g"], d["h0"], per_channel=True,
                               flags=drla.SERIAL)
    torch.cuda.synchronize()
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    del d
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o, o_ref), rel_err(ht, ht_ref)
    print(f"  rel_err o={eo:.3e} ht={eh:.3e} (tol {TOL['bf16']:g})", flush=True)
    assert np.isfinite(o).all() and eo <= TOL["bf16"] and eh <= TOL["bf16"]
