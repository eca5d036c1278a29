"""drla_prefill_noalloc (the entry point for callers that cannot allocate)
against gdn_prefill / kda_prefill with a workspace: the same kernels on the
same inputs, so the results must be identical.  Two calls in a row, the
second with a smaller input, and each call checked against the oracle to
the parity bar as well."""
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


def _both(drla, x):
    d = to_device(x)
    kda = x["kind"] == "kda"
    fn = drla.kda_prefill if kda else drla.gdn_prefill
    o1, h1 = fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                cu_seqlens_host=d["cu_host"])
    o2, h2 = drla.prefill_noalloc(kda, d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"],
                                  d["cu"], cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (o1, h1, o2, h2)]


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_noalloc_matches_workspace_call(drla, kind):
    big = W.small_spec(kind, lens=(700, 130, 65, 1), h_qk=2, h_v=4, dk=128, dv=128, io="bf16",
                       g_lo=0.01, g_hi=0.2, h0_std=0.02, seed=21)
    small = W.small_spec(kind, lens=(150,), h_qk=1, h_v=2, dk=64, dv=128, io="bf16",
                         g_lo=0.01, g_hi=0.2, h0_std=0.02, seed=22)
    for tag, spec in (("first (larger)", big), ("second (smaller)", small)):
        x = W.make_inputs(spec)
        print(f"noalloc {kind} {tag}: lens={spec.lens[:4]} h_v={spec.h_v} dk={spec.dk}", flush=True)
        o1, h1, o2, h2 = _both(drla, x)
        np.testing.assert_array_equal(o2, o1)
        np.testing.assert_array_equal(h2, h1)
        o_ref, h_ref = run_oracle(x)
        eo, eh = rel_err(o2, o_ref), rel_err(h2, h_ref)
        print(f"noalloc {kind} {tag}: identical to the workspace call; rel_err o={eo:.2e} "
              f"ht={eh:.2e}", flush=True)
        assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_noalloc_rejects_oversize(drla):
    """A call whose workspace exceeds the scratch array is refused before
    anything is launched (32,768 tokens x 16 heads needs more than 64 MiB)."""
    T, H, d = 32768, 16, 128
    need = drla.workspace_bytes((T, H, d), (T, H, d))
    assert need > drla.NOALLOC_SCRATCH_BYTES
    dev = "cuda:0"
    q = torch.zeros((T, H, d), dtype=torch.bfloat16, device=dev)
    beta = torch.zeros((T, H), dtype=torch.float32, device=dev)
    g = torch.zeros((T, H), dtype=torch.float32, device=dev)
    with pytest.raises(drla.DrlaError, match="scratch"):
        drla.prefill_noalloc(False, q, q.clone(), q.clone(), beta, g)
