"""Shared helpers for the tests: tensors from the seeded generator, error
metrics, and decoding of the workspace's fragment order.  No arithmetic of
the method lives here."""
import numpy as np

# Max-norm relative error bounds per io dtype, for o and the final state.
# bf16 and fp32 bars as stated for the method; fp16 (no stated bar): about
# ten units in the last place of fp16 (2^-11), where the bf16 bar is about
# five of bf16 (2^-8)
TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-4}


def rel_err(x, y):
    """max|x - y| / max|y| (y = oracle)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.abs(y).max() if y.size else 0.0
    if den == 0.0:
        return float(np.abs(x).max()) if x.size else 0.0
    return float(np.abs(x - y).max() / den)


def nmse(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = float((y * y).sum())
    return float(((x - y) ** 2).sum() / d) if d > 0 else float((x * x).sum())


def to_device(x, device="cuda"):
    """Generator output (numpy) -> device tensors in the io dtype."""
    import torch
    io = {"bf16": torch.bfloat16, "f16": torch.float16}.get(x["io"], torch.float32)
    d = {}
    for name in ("q", "k", "v"):
        d[name] = torch.from_numpy(np.ascontiguousarray(x[name])).to(device=device, dtype=io)
    for name in ("beta", "g"):
        d[name] = torch.from_numpy(np.ascontiguousarray(x[name])).to(device=device)
    d["h0"] = None if x["h0"] is None else torch.from_numpy(x["h0"]).to(device=device)
    if x["varlen"]:
        d["cu"] = torch.from_numpy(x["cu_seqlens"]).to(device=device)
        d["cu_host"] = [int(c) for c in x["cu_seqlens"]]
    else:
        d["cu"] = None
        d["cu_host"] = None
    return d


def run_oracle(x, heads=None, threads=None):
    """fp64 oracle on the same (bf16-rounded) inputs; optionally only the
    listed v-heads (returns arrays for those heads only)."""
    import oracle
    q, k, v, beta, g, h0 = x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"]
    if heads is not None:
        grp = x["h_v"] // x["h_qk"]
        hk = [h // grp for h in heads]
        q, k = q[:, hk], k[:, hk]
        v, beta, g = v[:, heads], beta[:, heads], g[:, heads]
        h0 = None if h0 is None else h0[:, heads]
    cu = x["cu_seqlens"] if x["varlen"] else None
    if x["kind"] in ("ret", "gla"):  # decay-only linear attention
        return oracle.recurrence_decay(q, k, v, g, h0, cu, per_channel=x["kind"] == "gla")
    return oracle.recurrence(q, k, v, beta, g, h0, cu, kda=x["kind"] == "kda",
                             threads=threads)


def kmap(g, j):
    """Inner index of slot j in lane group g (the fragment order of the
    library's workspace: 4 + 4 at a distance of 16)."""
    return 4 * g + j if j < 4 else 16 + 4 * g + (j - 4)


def kmap_contiguous(g, j):
    """Inner index of slot j in lane group g for fragments whose inner index
    is a key channel (8 contiguous channels per lane)."""
    return 8 * g + j


def _slot_index(inner_map):
    """(lane, j) -> (outer offset 0..15, inner offset 0..31) of a fragment."""
    outer = np.zeros((64, 8), dtype=np.int64)
    inner = np.zeros((64, 8), dtype=np.int64)
    for lane in range(64):
        for j in range(8):
            outer[lane, j] = lane % 16
            inner[lane, j] = inner_map(lane // 16, j)
    return outer, inner


def decode_blocks(raw, n_outer, n_inner, order, inner_map=kmap):
    """Decode one (v-head, chunk) region stored as fragments.

    raw        flat array of n_outer*n_inner elements
    order      "outer_major": fragment index = tile*(n_inner/32) + p
    inner_map  slot -> inner index map (kmap or kmap_contiguous)
    returns    dense [n_outer, n_inner] (outer index, inner index)
    """
    assert order == "outer_major"
    to, ti = _slot_index(inner_map)
    nb_in = n_inner // 32
    dense = np.zeros((n_outer, n_inner), dtype=np.float64)
    blocks = np.asarray(raw, dtype=np.float64).reshape(-1, 64, 8)
    for b in range(blocks.shape[0]):
        tile, p = divmod(b, nb_in)
        dense[16 * tile + to, 32 * p + ti] = blocks[b]
    return dense


def state_row(mt, rho):
    """Key channel held by row rho of state tile mt in the scan kernel."""
    return 32 * (mt >> 1) + 8 * (rho >> 2) + 4 * (mt & 1) + (rho & 3)
