"""The library only enqueues kernels on the caller's stream (no allocation,
copy, fill or synchronisation), so a call can be captured into a HIP graph.
Each case captures one call, then replays the graph several times with
unrelated eager calls of the library and synchronisations between the
replays, and requires every replay to equal the eager result bit for bit
(the kernels are deterministic)."""
import pytest

import workloads as W
from drla_testlib import to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def drla():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import delta_rule_linear_chunked_amd as m
    m.load_library()
    return m


def _inputs(kind, lens, io="bf16", seed=21):
    g_lo, g_hi = (0.01, 0.2) if kind == "gdn" else (0.005, 0.15)
    s = W.small_spec(kind, lens=lens, h_qk=2, h_v=4, dk=128, dv=128, io=io, g_lo=g_lo,
                     g_hi=g_hi, h0_std=0.05, seed=seed)
    return to_device(W.make_inputs(s))


def _replay_and_compare(call, other):
    o_e, ht_e = call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, ht_g = call()
    for r in range(4):
        other()                      # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(ht_g, ht_e), f"replay {r}"


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("lens", [(300,), (130, 0, 257, 64)])
def test_prefill_graph_replays(drla, kind, lens):
    print(f"case graph prefill kind={kind} lens={lens}", flush=True)
    d = _inputs(kind, lens)
    e = _inputs(kind, (200, 90), seed=22)
    fn = drla.kda_prefill if kind == "kda" else drla.gdn_prefill

    def call():
        return fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"], d["cu"],
                  cu_seqlens_host=d["cu_host"])

    def other():
        fn(e["q"], e["k"], e["v"], e["beta"], e["g"], e["h0"], e["cu"],
           cu_seqlens_host=e["cu_host"])

    _replay_and_compare(call, other)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_decode_graph_replays(drla, kind):
    print(f"case graph decode kind={kind}", flush=True)
    d = _inputs(kind, (1,) * 8)
    e = _inputs(kind, (1,) * 5, seed=23)
    fn = drla.kda_decode if kind == "kda" else drla.gdn_decode

    def call():
        return fn(d["q"], d["k"], d["v"], d["beta"], d["g"], d["h0"])

    def other():
        fn(e["q"], e["k"], e["v"], e["beta"], e["g"], e["h0"])

    _replay_and_compare(call, other)
