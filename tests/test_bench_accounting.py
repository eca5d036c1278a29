"""The byte counts behind bench.py's roofline figures, against per-token
figures worked out from the tensors the method reads and writes (CPU only).

Per token and value head, bf16 q/k/v with as many q/k heads as value heads
and dk = dv = 128: q and k 2 x 128 x 2 B, v 128 x 2 B, o 128 x 2 B, beta
4 B, and the log-gate 4 B (GDN, one per token and head) or 128 x 4 B (KDA,
one per key channel): 1,032 B for GDN and 1,540 B for KDA.  Each (sequence,
head) adds its fp32 128 x 128 state once out (ht) and once in when h0 is
given: 65,536 B each."""
import bench
import workloads as W

STATE = 128 * 128 * 4


def test_whole_call_bytes_gdn_prefill():
    s = W.WORKLOADS["gdn_prefill"]                     # zero initial state
    assert bench.call_io_bytes(s, 4096, 1) == 4096 * 16 * 1032 + 16 * STATE


def test_whole_call_bytes_kda_prefill():
    s = W.WORKLOADS["kda_prefill"]                     # nonzero initial state
    assert bench.call_io_bytes(s, 4096, 1) == 4096 * 16 * 1540 + 2 * 16 * STATE


def test_whole_call_bytes_grouped_varlen():
    # 16 q/k heads shared by 32 value heads: q and k are read once per q/k head
    s = W.WORKLOADS["gdn_varlen"]
    T = sum(s.lens)
    per_token = 2 * 16 * 128 * 2 + 32 * (128 * 2 * 2 + 4 + 4)
    assert bench.call_io_bytes(s, T, 8) == T * per_token + 2 * 8 * 32 * STATE


def test_scan_kernel_bytes_leave_out_beta():
    # the scan reads q, k, v and the scalar gate, writes o and ht; beta is
    # prep's alone: 1,028 B per token-head at gdn_prefill
    s = W.WORKLOADS["gdn_prefill"]
    scan_bytes, _ = bench.kernel_costs(s, 4096, 1)["scan"]
    assert scan_bytes == 4096 * 16 * 1028 + 16 * STATE
