"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle/recurrence.c is built with gcc -fsanitize=address,undefined (no
recovery: the first report aborts) together with a driver that gives every
array an allocation of its exact size, and runs on packed ragged inputs that
reach its edge cases: an empty sequence, a one-token sequence, grouped heads,
dk != dv, no initial state, more threads than (sequence, head) units.  The
sanitized results must also equal those of the regular build."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")
SOURCE = os.path.join(ROOT, "oracle", "recurrence.c")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("asan") / "oracle_asan")
    subprocess.check_call([gcc, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-pthread", DRIVER, SOURCE, "-lm", "-o", exe])
    return exe


CASES = [
    # mode, kind, lens, h_qk, h_v, dk, dv, h0_std, threads
    ("delta", "gdn", (37, 0, 1, 70), 1, 2, 16, 24, 0.1, 3),
    ("delta", "kda", (5, 66, 0), 2, 4, 24, 8, 0.0, 16),
    ("delta", "gdn", (0,), 1, 1, 8, 8, 0.1, 2),
    ("decay", "ret", (9, 0, 40), 1, 2, 16, 8, 0.1, 1),
    ("decay", "gla", (1, 33), 2, 2, 8, 16, 0.0, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[1]}-{len(c[2])}seq")
def test_oracle_clean_under_asan_ubsan(sanitized, tmp_path, case):
    mode, kind, lens, h_qk, h_v, dk, dv, h0_std, threads = case
    x = W.make_inputs(W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv,
                                   io="f32", h0_std=h0_std, seed=5, varlen=True))
    per_channel = kind in ("kda", "gla")
    cu = np.asarray(x["cu_seqlens"], dtype=np.int64)
    n, T = len(cu) - 1, int(cu[-1])
    f64 = lambda a: np.ascontiguousarray(a, dtype=np.float64)  # noqa: E731
    hd = np.array([0 if mode == "delta" else 1, int(per_channel), n, h_qk, h_v, dk, dv, T,
                   int(x["h0"] is not None), threads], dtype=np.int64)
    parts = [hd, cu, f64(x["q"]), f64(x["k"]), f64(x["v"])]
    if mode == "delta":
        parts.append(f64(x["beta"]))
    parts.append(f64(x["g"]))
    if x["h0"] is not None:
        parts.append(f64(x["h0"]))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for p in parts:
            f.write(p.tobytes())
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized, str(src), str(dst)], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    out = np.fromfile(dst, dtype=np.float64)
    no = T * h_v * dv
    o_s, ht_s = out[:no].reshape(T, h_v, dv), out[no:].reshape(n, h_v, dk, dv)
    cuv = x["cu_seqlens"]
    if mode == "delta":
        o_r, ht_r = oracle.recurrence(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"], cuv,
                                      kda=per_channel, threads=threads)
    else:
        o_r, ht_r = oracle.recurrence_decay(x["q"], x["k"], x["v"], x["g"], x["h0"], cuv,
                                            per_channel=per_channel)
    np.testing.assert_allclose(o_s, o_r, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht_s, ht_r, rtol=1e-12, atol=1e-12)
