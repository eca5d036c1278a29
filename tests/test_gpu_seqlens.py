"""The host/device cu_seqlens contract of packed calls (GPU).

The host copy of the lengths is validated and sizes the launch and the
workspace; the kernels take the device copy, which the first kernel checks
against the host's (cu[0] = 0, non-decreasing, cu[N] = T, chunk counts, a
64-bit fingerprint of every entry) before any kernel reads a token.  When
they agree the call is the ordinary one (checked against the oracle).  When
they differ -- other lengths with the same total, a total past the end of
the inputs, a decreasing entry -- the call runs as N empty sequences: o is
left as it was, every final state is its initial state, and
drla_prefill_status reports DRLA_ERR_SEQLENS (verify_lengths raises).  The
next agreeing call on the same workspace reports DRLA_OK again."""
import numpy as np
import pytest

import workloads as W
from drla_testlib import TOL, rel_err, run_oracle, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SEQLENS_ERR = 5  # DRLA_ERR_SEQLENS


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _inputs(kind, lens, io="bf16"):
    return W.make_inputs(W.small_spec(kind, lens=lens, h_qk=1, h_v=2, dk=128, dv=128, io=io,
                                      g_lo=0.01, g_hi=0.2, h0_std=0.05, seed=23, varlen=True))


def _run(drla, kind, d, cu_dev, cu_host, o, ht, ws, flags=0, verify=True):
    fn = drla.kda_prefill if kind == "kda" else drla.gdn_prefill
    return fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], cu_dev, cu_seqlens_host=cu_host,
              out=o, final_state=ht, workspace=ws, flags=flags, verify_lengths=verify)


def _buffers(drla, x, d, cu_host, flags):
    T, n = int(x["cu_seqlens"][-1]), len(cu_host) - 1
    lay = drla.workspace_layout(d["q"].shape, d["v"].shape, d["q"].dtype, n_seqs=n,
                                cu_seqlens_host=cu_host, kda=x["kind"] == "kda", flags=flags)
    ws = torch.empty(max(int(lay["total"]), 1), dtype=torch.uint8, device="cuda")
    o = torch.full((T, x["h_v"], 128), 7.0, dtype=d["q"].dtype, device="cuda")
    ht = torch.empty((n, x["h_v"], 128, 128), dtype=torch.float32, device="cuda")
    return ws, o, ht


# device copies of host lengths [0, 100, 300] (2 + 4 chunks)
BAD = {
    "same-total": [0, 150, 300],      # 3 + 3 chunks: only the fingerprint differs
    "past-the-end": [0, 100, 5000],   # tokens past the end of q, k, v
    "decreasing": [0, 350, 300],
    "nonzero-start": [64, 100, 300],
}


@pytest.mark.parametrize("kind,flag", [("gdn", 0), ("gdn", "HEAD_SCAN"), ("gdn", "SERIAL"),
                                       ("kda", 0)])
@pytest.mark.parametrize("bad", sorted(BAD))
def test_mismatched_lengths_run_empty_and_report(drla, kind, flag, bad):
    print(f"case seqlens {kind} flag={flag} device={bad}", flush=True)
    flags = getattr(drla, flag) if flag else 0
    x = _inputs(kind, (100, 200))
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    ws, o, ht = _buffers(drla, x, d, cu_host, flags)
    cu_bad = torch.tensor(BAD[bad], dtype=torch.int32, device="cuda")
    with pytest.raises(drla.DrlaError) as err:
        _run(drla, kind, d, cu_bad, cu_host, o, ht, ws, flags)
    assert err.value.status == SEQLENS_ERR
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "o was written"
    np.testing.assert_array_equal(ht.cpu().numpy(), x["h0"])
    # the same workspace, agreeing lengths: the ordinary call, status OK
    o2, ht2 = _run(drla, kind, d, d["cu"], cu_host, None, None, ws, flags)
    o_ref, ht_ref = run_oracle(x)
    eo = rel_err(o2.float().cpu().numpy(), o_ref)
    eh = rel_err(ht2.cpu().numpy(), ht_ref)
    print(f"seqlens {kind}/{bad}: agreeing call rel_err o={eo:.3e} ht={eh:.3e}", flush=True)
    assert eo <= TOL[x["io"]] and eh <= TOL[x["io"]]


def test_mismatch_without_verify_returns_ok_and_status_reports_it(drla):
    """The call itself is asynchronous and returns DRLA_OK; the status call
    afterwards reports the mismatch."""
    x = _inputs("gdn", (100, 200))
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    ws, o, ht = _buffers(drla, x, d, cu_host, 0)
    cu_bad = torch.tensor(BAD["same-total"], dtype=torch.int32, device="cuda")
    call = drla.prepare_prefill(False, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], cu_bad,
                                cu_seqlens_host=cu_host, workspace=ws, out=o, final_state=ht)
    call()
    with pytest.raises(drla.DrlaError) as err:
        call.check_lengths()
    assert err.value.status == SEQLENS_ERR


def test_noalloc_reports_mismatch(drla):
    x = _inputs("gdn", (100, 200))
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    cu_bad = torch.tensor(BAD["past-the-end"], dtype=torch.int32, device="cuda")
    with pytest.raises(drla.DrlaError) as err:
        drla.prefill_noalloc(False, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], cu_bad,
                             cu_host, verify_lengths=True)
    assert err.value.status == SEQLENS_ERR
    o, ht = drla.prefill_noalloc(False, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                                 cu_host, verify_lengths=True)
    o_ref, _ = run_oracle(x)
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL[x["io"]]


def test_many_sequences_fingerprint(drla):
    """700 packed sequences (the schedule kernel's threads each fold several
    entries into the fingerprint): agreeing lengths pass, one entry moved by
    one token fails."""
    rng = np.random.default_rng(3)
    lens = tuple(int(v) for v in rng.integers(0, 40, size=700))
    x = _inputs("gdn", lens)
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    ws, o, ht = _buffers(drla, x, d, cu_host, 0)
    _run(drla, "gdn", d, d["cu"], cu_host, o, ht, ws)
    o_ref, _ = run_oracle(x)
    assert rel_err(o.float().cpu().numpy(), o_ref) <= TOL[x["io"]]
    moved = list(cu_host)
    i = next(j for j in range(1, 700) if moved[j - 1] < moved[j] - 1 and moved[j] < moved[j + 1])
    moved[i] -= 1  # same chunk total unless a boundary is crossed; the fingerprint differs
    with pytest.raises(drla.DrlaError):
        _run(drla, "gdn", d, torch.tensor(moved, dtype=torch.int32, device="cuda"), cu_host, o, ht, ws)


@pytest.mark.parametrize("n", [1024, 1025, 3000])
def test_batches_past_the_lds_table(drla, n):
    """The schedule kernel keeps the lengths of batches of up to 1,024
    sequences in LDS (the chunk table written by every thread, the ranking
    done there); larger batches take the per-sequence table writes and the
    separate ranking kernel.  Both sides of the limit, against the oracle."""
    rng = np.random.default_rng(n)
    lens = tuple(int(v) for v in rng.integers(0, 90, size=n))
    x = _inputs("gdn", lens)
    d = to_device(x)
    cu_host = [int(c) for c in x["cu_seqlens"]]
    o, ht = _run(drla, "gdn", d, d["cu"], cu_host, None, None, None)
    o_ref, ht_ref = run_oracle(x)
    eo, eh = rel_err(o.float().cpu().numpy(), o_ref), rel_err(ht.cpu().numpy(), ht_ref)
    print(f"batch of {n}: rel_err o={eo:.3e} ht={eh:.3e}", flush=True)
    assert eo <= TOL[x["io"]] and eh <= TOL[x["io"]]
