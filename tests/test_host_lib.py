"""CPU tests of the C ABI library: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU (the validation
path makes no HIP call, so it runs without a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "drla.h")


@pytest.fixture(scope="module")
def lib():
    from delta_rule_linear_chunked_amd import _lib
    if not os.path.exists(_lib.lib_path()):
        from delta_rule_linear_chunked_amd import build
        build.build()
    return _lib.load_library()


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert {"gdn_prefill", "kda_prefill", "gdn_decode", "kda_decode", "drla_prefill_ex",
            "drla_workspace_bytes", "drla_workspace_layout", "drla_status_str", "drla_last_error",
            "drla_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.drla_version() == 7


def test_prefill_status_needs_no_device_for_unpacked_calls(lib):
    """drla_prefill_status: a dense call (no cu_seqlens) or one packed
    sequence reads no device lengths, so it is DRLA_OK without a device; a
    malformed problem is refused."""
    p = _prob(n_seqs=1, T=256)
    assert lib.drla_prefill_status(ctypes.byref(p), None, None, None) == 0
    cu, keep = _i32([0, 256])
    assert lib.drla_prefill_status(ctypes.byref(p), cu, None, None) == 0
    bad = _prob(n_seqs=2, T=256)
    cu2, keep2 = _i32([0, 300, 256])
    assert lib.drla_prefill_status(ctypes.byref(bad), cu2, None, None) == 5


def test_peaks_library_exports_its_header():
    """libdrla_peaks.so (the benchmark's attainable-peak kernels) exports
    what include/drla_peaks.h declares and refuses bad arguments before any
    launch."""
    from delta_rule_linear_chunked_amd import build
    if not os.path.exists(build.PEAKS_LIB):
        build.build()
    peaks = ctypes.CDLL(build.PEAKS_LIB)
    names = _declared_functions(os.path.join(ROOT, "include", "drla_peaks.h"))
    assert set(names) == {"drla_peak_copy", "drla_peak_mfma", "drla_peak_mfma_grid"}
    for n in names:
        assert hasattr(peaks, n), n
    peaks.drla_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    base = 1 << 40
    assert peaks.drla_peak_copy(base, base + (1 << 30), 100, None) == 1   # not a multiple of 16
    assert peaks.drla_peak_copy(base, base + 64, 128, None) == 1          # overlapping
    assert peaks.drla_peak_copy(base + 8, base + (1 << 30), 128, None) == 1  # misaligned
    assert peaks.drla_peak_copy(None, base, 128, None) == 1
    peaks.drla_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert peaks.drla_peak_mfma(base, 3, 10, 1, None, None, None) == 1       # unknown kind
    assert peaks.drla_peak_mfma(base, 0, 0, 1, None, None, None) == 1        # no iterations
    assert peaks.drla_peak_mfma_grid(7) == 7


def _prob(n_seqs=1, h_qk=2, h_v=4, dk=128, dv=128, io=0, T=256):
    from delta_rule_linear_chunked_amd._lib import Problem
    return Problem(n_seqs, h_qk, h_v, dk, dv, io, T)


def _call(lib, p, q=16, ws=16, cu_dev=None, cu_host=None, h0=None, ht=None, o=1 << 20,
          kda=False, ws_bytes=1 << 40):
    # Fake, aligned, non-overlapping "device" addresses: validation only
    # compares and checks them; it never dereferences them.
    base = 1 << 40
    args = [ctypes.byref(p), base + q * 0 + 0x1000000 if q else None, base + 0x2000000,
            base + 0x3000000, base + 0x4000000, base + 0x5000000, h0, cu_dev,
            cu_host, base + o + 0x6000000 if o else None, ht,
            base + 0x70000000 if ws else None, ws_bytes, None]
    fn = lib.kda_prefill if kda else lib.gdn_prefill
    return fn(*args)


def _i32(vals):
    arr = (ctypes.c_int32 * len(vals))(*vals)
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), arr


def test_validation_errors(lib):
    assert lib.gdn_prefill(None, None, None, None, None, None, None, None, None, None,
                           None, None, 0, None) == 1
    assert _call(lib, _prob(h_v=3)) == 2               # h_v % h_qk
    assert _call(lib, _prob(dk=96)) == 3               # unsupported dk
    assert _call(lib, _prob(io=7)) == 3                # unknown dtype
    assert _call(lib, _prob(n_seqs=3, T=256)) == 2     # T % N for a dense batch
    assert _call(lib, _prob(), q=0) == 1               # null q
    assert _call(lib, _prob(), ws=0) == 6              # no workspace
    assert _call(lib, _prob(), ws_bytes=10) == 6       # workspace too small
    # misaligned pointer
    p = _prob()
    assert lib.gdn_prefill(ctypes.byref(p), (1 << 40) + 2, 1 << 41, 1 << 42, 1 << 43,
                           1 << 44, None, None, None, 1 << 45, None, 1 << 46, 1 << 40, None) == 4
    # output overlapping an input
    assert lib.gdn_prefill(ctypes.byref(p), 1 << 40, 1 << 41, 1 << 42, 1 << 43,
                           1 << 44, None, None, None, 1 << 40, None, 1 << 46, 1 << 40, None) == 7
    msg = lib.drla_last_error().decode()
    assert "overlap" in msg


def test_decode_validation_errors(lib):
    """The decode entry points check everything before enqueueing anything
    (fake aligned addresses: never dereferenced on these paths)."""
    b = 1 << 40
    ins = [b + 0x1000000, b + 0x2000000, b + 0x3000000, b + 0x4000000, b + 0x5000000]

    def call(p, q=ins[0], h0=None, o=b + 0x6000000, ht=b + 0x7000000, kda=False):
        fn = lib.kda_decode if kda else lib.gdn_decode
        return fn(ctypes.byref(p), q, *ins[1:], h0, o, ht, None)

    assert lib.gdn_decode(None, *([None] * 9)) == 1
    assert call(_prob(n_seqs=4, T=8)) == 2              # two tokens per sequence
    assert call(_prob(n_seqs=4, T=4, h_v=3)) == 2       # h_v % h_qk
    assert call(_prob(n_seqs=4, T=4, dk=96)) == 3       # unsupported dk
    assert call(_prob(n_seqs=4, T=4), q=None) == 1      # null q
    assert call(_prob(n_seqs=4, T=4), o=None) == 1      # null o
    assert call(_prob(n_seqs=4, T=4), q=ins[0] + 8) == 4, "misaligned q"
    assert call(_prob(n_seqs=4, T=4), o=ins[2], kda=True) == 7   # o over v
    assert call(_prob(n_seqs=4, T=4), h0=b + 0x8000000, ht=b + 0x8000000 + 4096) == 7
    assert "overlap" in lib.drla_last_error().decode()


def test_decay_entry_points_validate(lib):
    """decay_prefill / decay_decode take no beta and check the rest as the
    delta-rule calls do (fake aligned addresses, never dereferenced)."""
    b = 1 << 40
    p = _prob(n_seqs=1, T=256)
    args = [b + 0x1000000, b + 0x2000000, b + 0x3000000, b + 0x4000000, None, None, None,
            b + 0x6000000, None, b + 0x70000000, 1 << 40, None]
    assert lib.decay_prefill(0, ctypes.byref(p), None, *args[1:]) == 1      # null q
    assert lib.decay_prefill(0, ctypes.byref(_prob(dk=96)), *args) == 3   # unsupported dk
    assert lib.decay_prefill(1, ctypes.byref(p), *args[:9], 0, 0, None) == 6  # no workspace
    pd = _prob(n_seqs=4, T=4)
    assert lib.decay_decode(0, ctypes.byref(pd), b, b + 0x100000, b + 0x200000, None,
                            None, b + 0x300000, None, None) == 1       # null g
    assert lib.decay_decode(1, ctypes.byref(_prob(n_seqs=4, T=8)), b, b + 0x100000, b + 0x200000,
                            b + 0x400000, None, b + 0x300000, None, None) == 2


def test_cu_seqlens_validation(lib):
    p = _prob(n_seqs=3, T=100)
    dev = ctypes.cast(ctypes.c_void_p(1 << 47), ctypes.POINTER(ctypes.c_int32))
    good, _g = _i32([0, 30, 30, 100])
    assert _call(lib, p, cu_dev=dev, cu_host=None) == 5          # only one of the pair
    bad0, _b0 = _i32([1, 30, 40, 100])
    assert _call(lib, p, cu_dev=dev, cu_host=bad0) == 5
    dec, _d = _i32([0, 40, 30, 100])
    assert _call(lib, p, cu_dev=dev, cu_host=dec) == 5
    end, _e = _i32([0, 30, 40, 99])
    assert _call(lib, p, cu_dev=dev, cu_host=end) == 5
    # the valid one gets past validation and fails only for the workspace size
    assert _call(lib, p, cu_dev=dev, cu_host=good, ws_bytes=1) == 6


def test_workspace_bytes_and_layout(lib):
    from delta_rule_linear_chunked_amd._lib import Layout
    p = _prob(n_seqs=1, h_qk=16, h_v=16, dk=128, dv=128, io=0, T=4096)
    n = lib.drla_workspace_bytes(ctypes.byref(p), None)
    lay = Layout()
    assert lib.drla_workspace_layout(1, ctypes.byref(p), None, 0, ctypes.byref(lay)) == 0
    assert lay.n_chunks == 64
    per = 64 * 16                       # (chunk, head) pairs
    frag = 64 * 8 * 2                   # one bf16 fragment
    assert lay.pm - lay.tb == per * 8 * frag
    assert lay.kt - lay.pm == per * 8 * frag
    assert lay.kw - lay.kt == per * 64 * 128 * 2
    assert lay.qw - lay.kw == per * 64 * 128 * 2
    assert lay.gam - lay.qw == per * 64 * 128 * 2
    assert lay.total - lay.gam == per * 128 * 4
    assert lay.vp == 0 and lay.h == 0 and lay.seg == 0   # 16 x 8 blocks: no segment split
    # GDN with bf16 inputs needs neither K~^T nor the KDA operands; its decay
    # factors are 2 x 64 floats per chunk
    gl = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 0, ctypes.byref(gl)) == 0
    assert gl.kt == 0 and gl.kw == 0 and gl.qw == 0 and gl.gam == lay.kt
    # its scan pairs a later segment's two chains in one workgroup: 16 heads
    # x 8 column blocks x 2 segments fill 256 compute units
    us = 16 * 128 * 128
    assert gl.hs == 0 and gl.seg >= gl.gam + per * 128 * 4
    assert gl.total - gl.seg == us * 4 + 2 * us * 4 + us * 2 + 4096 * 16 * 128 * 2
    assert n == max(lay.total, gl.total)
    # with DRLA_HEAD_SCAN (8): the head-resident scan splits 16 units into 16
    # segments of 4 chunks: 15 fp32 state sets and 14 bf16 segment maps per unit
    hl = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 8, ctypes.byref(hl)) == 0
    assert hl.seg == 0 and hl.hs == hl.gam + per * 128 * 4
    assert hl.total - hl.hs == 15 * 16 * 128 * 128 * 4 + 14 * 16 * 128 * 128 * 2
    # 8 heads (8 x 8 column blocks x 3 <= 256 CUs; 32 chunks per segment:
    # not paired): three fp32 states per head, the first as bf16 fragments,
    # and G laid out like o
    p8 = _prob(n_seqs=1, h_qk=8, h_v=8, dk=128, dv=128, io=0, T=4096)
    sl = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p8), None, 0, ctypes.byref(sl)) == 0
    assert sl.seg - sl.gam == 64 * 8 * 128 * 4 and sl.hs == 0
    assert sl.total - sl.seg == 3 * 8 * 128 * 128 * 4 + 8 * 128 * 128 * 2 + 4096 * 8 * 128 * 2
    # 2 heads: paired, 16 segments of 16 workgroups (unpaired: 8 segments of
    # 128 chunks); fifteen N, M and fragment sets
    p2h = _prob(n_seqs=1, h_qk=2, h_v=2, dk=128, dv=128, io=0, T=65536)
    assert lib.drla_workspace_layout(0, ctypes.byref(p2h), None, 0, ctypes.byref(sl)) == 0
    us = 2 * 128 * 128
    assert sl.total - sl.seg == us * 4 + 15 * 2 * us * 4 + 15 * us * 2 + 65536 * 2 * 128 * 2
    # one sequence passed with cu_seqlens {0, T} is laid out as the dense call
    cu1, _c1 = _i32([0, 4096])
    for flags in (0, 8):
        dl, pl = Layout(), Layout()
        assert lib.drla_workspace_layout(0, ctypes.byref(p8), None, flags, ctypes.byref(dl)) == 0
        assert lib.drla_workspace_layout(0, ctypes.byref(p8), cu1, flags, ctypes.byref(pl)) == 0
        assert (pl.tb, pl.seg, pl.hs, pl.total) == (dl.tb, dl.seg, dl.hs, dl.total)
        assert (pl.hs if flags else pl.seg) > 0
    assert lib.drla_workspace_bytes(ctypes.byref(p8), cu1) == lib.drla_workspace_bytes(ctypes.byref(p8), None)
    # fp32 inputs keep K~^T for the register-fed scan
    pf = _prob(n_seqs=1, h_qk=16, h_v=16, dk=128, dv=128, io=1, T=4096)
    fl = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(pf), None, 0, ctypes.byref(fl)) == 0
    assert fl.gam - fl.kt == per * 64 * 128 * 4
    # with the inspection flag V' and h follow
    kl = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 1, ctypes.byref(kl)) == 0
    assert kl.vp == gl.seg and kl.h - kl.vp == per * 64 * 128 * 2
    assert kl.total - kl.h == per * 128 * 128 * 2
    assert kl.hs == 0 and kl.seg == 0   # intermediates: the per-16-column scan, one pass
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 4, ctypes.byref(kl)) == 0
    assert kl.hs == 0 and kl.seg == 0   # DRLA_SERIAL: one pass
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 32, ctypes.byref(kl)) == 3
    # 11 heads of 8 column blocks: 2 x 88 paired workgroups split (3 x 88 =
    # 264 unpaired ones would not fit: KDA keeps one pass)
    p11 = _prob(n_seqs=1, h_qk=11, h_v=11, dk=128, dv=128, io=0, T=4096)
    assert lib.drla_workspace_layout(0, ctypes.byref(p11), None, 0, ctypes.byref(kl)) == 0
    assert kl.seg > 0
    assert lib.drla_workspace_layout(1, ctypes.byref(p11), None, 0, ctypes.byref(kl)) == 0
    assert kl.seg == 0
    cu, _c = _i32([0, 1, 65, 65, 200])
    p2 = _prob(n_seqs=4, T=200)
    lay2 = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p2), cu, 0, ctypes.byref(lay2)) == 0
    assert lay2.n_chunks == 1 + 1 + 0 + 3
    assert lay2.tb >= (2 * 5 + 4 + 1) * 4      # chunk table first
    assert lay2.seg == 0 and lay2.hs == 0     # 3 chunks at most: one pass
    assert lib.drla_workspace_bytes(ctypes.byref(_prob(dk=80)), None) == 0


def test_status_strings(lib):
    for s in range(9):
        assert lib.drla_status_str(s)


def _seg_count(units_cb, max_cps, cus, paired):
    np_ = 1
    for p in range(2, 17):
        if (p if paired else 2 * p - 1) * units_cb <= cus and max_cps >= 4 * p:
            np_ = p
    return np_


def _seg_np(units_cb, max_cps, cus=256, can_pair=False):
    """The segment plan as the header states it: the most np <= 16 with
    (2 np - 1) U <= cus and at least 4 np chunks in the longest sequence; or,
    where pairing is possible, the most with np U <= cus when that is more
    and the unpaired split cannot run or leaves >= 96 chunks per segment."""
    nu = _seg_count(units_cb, max_cps, cus, False)
    npp = _seg_count(units_cb, max_cps, cus, True) if can_pair else 1
    return npp if npp > nu and (nu == 1 or max_cps // nu >= 96) else nu


SEG_SHAPES = [
    (1, 128, (3000,)), (2, 128, (65536,)), (4, 64, (8192,)), (8, 128, (4096,)),
    (11, 128, (4096,)), (1, 64, (1500,)), (2, 128, (1500, 700, 0, 2100)), (1, 128, (3000, 100, 0)),
    (4, 128, (200,)), (16, 64, (2000,)), (16, 128, (4096,)), (32, 128, (65536,)),
    (32, 128, (6745, 1169, 1890, 2330, 1905, 6666, 7188, 4983)),
]


@pytest.mark.parametrize("kda,io", [(0, 0), (1, 0), (1, 2), (0, 1), (1, 1)])
@pytest.mark.parametrize("h_v,d,lens", SEG_SHAPES)
def test_segment_region_follows_the_count_rule(lib, h_v, d, lens, kda, io):
    """The seg region (GDN and KDA, every io type) holds mid, np - 1 sets of
    N and M (fp32), np - 1 entering states in the io type, and G
    [T, h_v, d] in the io type.  Scalar-gate 16-bit calls pair a later
    segment's two chains in one workgroup, so they take more segments."""
    from delta_rule_linear_chunked_amd._lib import Layout
    n, T = len(lens), sum(lens)
    es = 4 if io == 1 else 2
    p = _prob(n_seqs=n, h_qk=1, h_v=h_v, dk=d, dv=d, io=io, T=T)
    cu, _c = _i32([0] + [sum(lens[:i + 1]) for i in range(n)])
    lay = Layout()
    assert lib.drla_workspace_layout(kda, ctypes.byref(p), cu if n > 1 else None, 0, ctypes.byref(lay)) == 0
    np_ = _seg_np(n * h_v * d // 16, max((L + 63) // 64 for L in lens), can_pair=(kda == 0 and io != 1))
    if np_ == 1:
        assert lay.seg == 0
        return
    us = n * h_v * d * d
    assert lay.seg > 0
    assert lay.total - lay.seg == us * 4 + 2 * (np_ - 1) * us * 4 + (np_ - 1) * us * es + T * h_v * d * es


@pytest.mark.parametrize("kda,io,h_v,d,T,flags,want", [
    (0, 0, 16, 128, 16384, 0, True),      # 16 heads, long: the head-resident scan
    (0, 2, 8, 128, 16384, 0, True),       # fp16, 8 heads
    (0, 0, 16, 128, 16384, 4, False),     # DRLA_SERIAL keeps the per-16-column scan
    (0, 0, 16, 128, 16384, 16, False),    # DRLA_COLUMN_SCAN keeps it too
    (0, 0, 16, 128, 4096, 0, False),      # short: per-16-column
    (0, 0, 32, 128, 65536, 0, False),     # 32 heads: per-16-column
    (0, 0, 2, 128, 65536, 0, False),      # 2 heads: the per-16-column split
    (1, 0, 16, 128, 16384, 0, False),     # KDA: per-16-column
    (0, 1, 16, 128, 16384, 0, False),     # fp32: per-16-column
    (0, 0, 16, 64, 16384, 0, False),      # d = 64: per-16-column
])
def test_automatic_head_scan_choice(lib, kda, io, h_v, d, T, flags, want):
    """Without flags, scalar-gate 16-bit calls at d = 128 take the
    head-resident scan where its timing model predicts it faster; the
    workspace layout records the choice (and holds the segmented head scan's
    region, no seg region)."""
    from delta_rule_linear_chunked_amd._lib import Layout
    p = _prob(n_seqs=1, h_qk=1, h_v=h_v, dk=d, dv=d, io=io, T=T)
    lay = Layout()
    assert lib.drla_workspace_layout(kda, ctypes.byref(p), None, flags, ctypes.byref(lay)) == 0
    assert lay.head_scan == int(want)
    assert (lay.hs > 0) == want
    if want:
        assert lay.seg == 0


def test_column_scan_flag(lib):
    """DRLA_COLUMN_SCAN keeps the per-16-column scan with its segment split
    where the model takes the head-resident scan; it excludes DRLA_HEAD_SCAN."""
    from delta_rule_linear_chunked_amd._lib import COLUMN_SCAN, HEAD_SCAN, Layout
    p = _prob(n_seqs=1, h_qk=1, h_v=8, dk=128, dv=128, io=0, T=65536)
    lay = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, 0, ctypes.byref(lay)) == 0
    assert lay.head_scan == 1 and lay.hs > 0 and lay.seg == 0
    assert lib.drla_workspace_layout(0, ctypes.byref(p), None, COLUMN_SCAN, ctypes.byref(lay)) == 0
    assert lay.head_scan == 0 and lay.hs == 0 and lay.seg > 0
    st = lib.drla_workspace_layout(0, ctypes.byref(p), None, COLUMN_SCAN | HEAD_SCAN, ctypes.byref(lay))
    assert st == 3  # DRLA_ERR_UNSUPPORTED
    assert b"exclude each other" in lib.drla_last_error()


def _model_choice(units, max_cps, unit_chunks, cus=256):
    """The scan-choice model as the header states it (dk = dv = 128)."""
    nh = _hs_np(units, max_cps, cus)
    if nh >= 3:
        t_head = 36 + 8.5 * -(-max_cps // nh)
    else:
        t_head = 4.07 * max(max_cps, unit_chunks / cus)
    chains = units * 8
    if chains > cus:
        t_col = 1.06 * max(max_cps, unit_chunks * 8 / cus)
    else:
        ns = _seg_np(chains, max_cps)
        t_col = 0.9 * -(-max_cps // ns) + (12 if ns > 1 else 0)
    return t_head < 0.9 * t_col


@pytest.mark.parametrize("lens,h_v,want", [
    ((1169, 2048, 3000, 4096, 5000, 6000, 7188, 4375), 32, True),  # packed, 2,048 chains: one-pass head scan
    ((4096,) * 8, 16, False),             # dense-like batch, 1,024 chains: near even, per-16-column
    ((2048,) * 32, 16, True),             # 32 sequences x 16 heads: the head scan's throughput wins
    ((7000, 100, 100, 100), 32, False),   # one long sequence dominates: per-16-column
    ((512,) * 64, 8, True),               # 512 short units
])
def test_automatic_choice_with_more_chains_than_compute_units(lib, lens, h_v, want):
    """Packed batches with more (unit, 16-column) chains than compute units:
    both scans are bound by the chunks each compute unit is dealt, and the
    head-resident one, which moves a chunk's operands once per head, is taken
    where the model predicts it at least 10 % faster.  The recorded choice
    follows the model as documented."""
    from delta_rule_linear_chunked_amd._lib import Layout
    n, T = len(lens), sum(lens)
    p = _prob(n_seqs=n, h_qk=h_v // 2, h_v=h_v, dk=128, dv=128, io=0, T=T)
    cu, _c = _i32([0] + [sum(lens[:i + 1]) for i in range(n)])
    lay = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), cu, 0, ctypes.byref(lay)) == 0
    cps = [(L + 63) // 64 for L in lens]
    assert _model_choice(n * h_v, max(cps), sum(cps) * h_v) == want
    assert lay.head_scan == int(want)
    if want:
        assert lay.seg == 0
    # DRLA_SERIAL keeps the per-16-column scan
    assert lib.drla_workspace_layout(0, ctypes.byref(p), cu, 4, ctypes.byref(lay)) == 0
    assert lay.head_scan == 0


def _hs_np(units, max_cps, cus=256):
    """The head-resident scan's segment count as the header states it: the
    most np with units x np <= cus, np^2 <= 9 n_max, at least two chunks per
    segment of the longest sequence and np <= 128; fewer than three: one
    pass."""
    np_ = min(cus // units, int((9 * max_cps) ** 0.5), max_cps // 2, 128)
    while (np_ + 1) ** 2 <= 9 * max_cps and np_ + 1 <= min(cus // units, max_cps // 2, 128):
        np_ += 1
    while np_ * np_ > 9 * max_cps:
        np_ -= 1
    return np_ if np_ >= 3 else 1


@pytest.mark.parametrize("h_v,d,lens", SEG_SHAPES)
def test_head_scan_region_follows_the_count_rule(lib, h_v, d, lens):
    """DRLA_HEAD_SCAN: the hs region holds np - 1 fp32 state sets and np - 2
    segment maps (dk x dk, bf16) per (sequence, head) unit."""
    from delta_rule_linear_chunked_amd._lib import Layout
    n, T = len(lens), sum(lens)
    p = _prob(n_seqs=n, h_qk=1, h_v=h_v, dk=d, dv=d, io=0, T=T)
    cu, _c = _i32([0] + [sum(lens[:i + 1]) for i in range(n)])
    lay = Layout()
    assert lib.drla_workspace_layout(0, ctypes.byref(p), cu if n > 1 else None, 8, ctypes.byref(lay)) == 0
    units = n * h_v
    np_ = _hs_np(units, max((L + 63) // 64 for L in lens))
    assert lay.seg == 0
    if np_ == 1:
        assert lay.hs == 0
        return
    assert lay.hs > 0
    assert lay.total - lay.hs == (np_ - 1) * units * d * d * 4 + (np_ - 2) * units * d * d * 2
    # dk != dv: one pass
    pq = _prob(n_seqs=n, h_qk=1, h_v=h_v, dk=d, dv=192 - d, io=0, T=T)
    assert lib.drla_workspace_layout(0, ctypes.byref(pq), cu if n > 1 else None, 8, ctypes.byref(lay)) == 0
    assert lay.hs == 0


def test_noalloc_rejects_oversize_before_the_device(lib):
    """drla_prefill_noalloc refuses a call whose workspace exceeds its
    scratch array (64 MiB) with DRLA_ERR_WORKSPACE, before any HIP call
    (fake aligned addresses, never dereferenced)."""
    b = 1 << 40
    p = _prob(n_seqs=1, h_qk=16, h_v=16, T=32768)
    args = [b + 0x1000000, b + 0x20000000, b + 0x40000000, b + 0x60000000, b + 0x70000000,
            None, None, None, b + 0x80000000, None, None]
    assert lib.drla_prefill_noalloc(0, 0, ctypes.byref(p), *args) == 6
    assert "scratch" in lib.drla_last_error().decode()
    # validation errors come first, as for the workspace call
    assert lib.drla_prefill_noalloc(0, 0, ctypes.byref(_prob(dk=96)), *args) == 3
