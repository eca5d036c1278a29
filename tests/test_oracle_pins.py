"""Pins for the fp64 oracle: facts fixed by the mathematics of the delta rule,
not by either oracle implementation.  Each test says which plausible mistake
it would catch.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(x, y):
    return np.abs(x - y).max() / max(np.abs(y).max(), 1e-300)


def _inputs(kind="gdn", lens=(37,), h_qk=1, h_v=1, dk=8, dv=5, h0_std=0.3,
            seed=0, g_lo=0.01, g_hi=0.2):
    s = W.small_spec(kind, lens=lens, h_qk=h_qk, h_v=h_v, dk=dk, dv=dv,
                     io="f32", g_lo=g_lo, g_hi=g_hi, h0_std=h0_std, seed=seed)
    return W.make_inputs(s)


def _run(x, fn=oracle.recurrence, **kw):
    kda = x["kind"] == "kda"
    return fn(x["q"], x["k"], x["v"], x["beta"], x["g"], x["h0"],
              x["cu_seqlens"] if x["varlen"] else None, kda=kda, **kw)


# ---- hand-worked example (exact values derived by hand) -------------------

def test_hand_worked_example():
    """Catches: output read from the pre-update state, a missing decay, beta
    on only the write or only the erase, a transposed state."""
    d = json.load(open(os.path.join(GOLDEN, "hand_worked.json")))
    q = np.array(d["q"])[:, None, :]
    k = np.array(d["k"])[:, None, :]
    v = np.array(d["v"])[:, None, :]
    beta = np.array(d["beta"])[:, None]
    g = np.log(np.array(d["alpha"]))[:, None]
    for fn in (oracle.recurrence, oracle.chunked):
        o, ht = fn(q, k, v, beta, g)
        np.testing.assert_allclose(o[:, 0, :], d["o"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(ht[0, 0], d["final_state"], rtol=0, atol=1e-15)


# ---- invariants -----------------------------------------------------------

@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_beta_zero_is_pure_decay(kind):
    """beta = 0: nothing is written, the state only decays:
    S_T = e^{sum g} S_0 (per key channel for KDA) and
    o_t = (e^{b_t} (.) S_0)^T q_t.  Catches a dropped/misplaced decay and a
    decay applied on the value index instead of the key index (dk != dv)."""
    x = _inputs(kind, lens=(23,), dk=6, dv=4)
    x["beta"][:] = 0.0
    o, ht = _run(x)
    G = np.cumsum(x["g"].astype(np.float64)[:, 0], axis=0)   # [T] or [T,dk]
    S0 = x["h0"][0, 0].astype(np.float64)
    q = x["q"][:, 0].astype(np.float64)
    if kind == "gdn":
        want_ht = np.exp(G[-1]) * S0
        want_o = np.exp(G)[:, None] * (q @ S0)
    else:
        want_ht = np.exp(G[-1])[:, None] * S0
        want_o = np.einsum("tc,tc,cj->tj", q, np.exp(G), S0)
    np.testing.assert_allclose(ht[0, 0], want_ht, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(o[:, 0], want_o, rtol=1e-12, atol=1e-15)
    # zero state with beta = 0 gives exactly zero output and state
    x["h0"] = None
    o, ht = _run(x)
    assert np.all(o == 0) and np.all(ht == 0)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_orthonormal_keys_are_recalled(kind):
    """alpha = 1, beta = 1, orthonormal keys k_1..k_n (n <= dk): the delta
    rule stores each pair exactly, S^T k_i = v_i, from any S_0, and leaves
    directions orthogonal to every key untouched.  Catches a wrong sign in
    the correction term, a missing erase (plain linear attention), and beta
    applied twice."""
    rng = np.random.default_rng(5)
    dk, dv, n = 12, 7, 9
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T                         # n orthonormal rows
    x = _inputs(kind, lens=(n,), dk=dk, dv=dv, h0_std=0.5)
    x["k"] = keys[:, None, :]
    x["g"][:] = 0.0
    x["beta"][:] = 1.0
    _, ht = _run(x)
    S = ht[0, 0]
    V = x["v"][:, 0].astype(np.float64)
    np.testing.assert_allclose(keys @ S, V, rtol=0, atol=1e-13)
    # the complement keeps S_0's action
    comp = Qm[:, n:].T
    np.testing.assert_allclose(comp @ S, comp @ x["h0"][0, 0], rtol=0, atol=1e-13)


def test_repeated_key_overwrites():
    """Same key written twice with beta = 1, alpha = 1: the second value
    replaces the first, S^T k = v_2 (linear attention would give v_1 + v_2)."""
    x = _inputs("gdn", lens=(2,), dk=5, dv=3, h0_std=0.0)
    k = x["k"][0, 0].astype(np.float64)
    k /= np.linalg.norm(k)               # exactly unit in fp64
    x["k"] = np.stack([k, k])[:, None, :]
    x["g"][:] = 0.0
    x["beta"][:] = 1.0
    _, ht = _run(x)
    np.testing.assert_allclose(k @ ht[0, 0], x["v"][1, 0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_basis_key_interpolates_row(kind):
    """One token with key e_0: row 0 of the state becomes the beta-weighted
    mix (1 - beta) * alpha_0 * S_0[0] + beta * v, and every other row j only
    decays (alpha_j S_0[j]).  With KDA the decay is applied before the write
    (so the write is not decayed), per key channel.  Catches the decay placed
    after the write, and beta misplaced between erase and write."""
    dk, dv = 6, 4
    x = _inputs(kind, lens=(1,), dk=dk, dv=dv, h0_std=0.7, g_lo=0.1, g_hi=0.9)
    x["k"][:] = 0.0
    x["k"][0, 0, 0] = 1.0
    b = float(x["beta"][0, 0])
    S0 = x["h0"][0, 0].astype(np.float64)
    if kind == "gdn":
        a = np.full(dk, np.exp(float(x["g"][0, 0])))
    else:
        a = np.exp(x["g"][0, 0].astype(np.float64))
    _, ht = _run(x)
    S1 = ht[0, 0]
    np.testing.assert_allclose(S1[0], (1 - b) * a[0] * S0[0] + b * x["v"][0, 0].astype(np.float64), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S1[1:], a[1:, None] * S0[1:], rtol=1e-14, atol=1e-15)


def test_output_reads_updated_state():
    """Zero state, one token: o_1 = beta (q . k) v, because the output is read
    from the state after this token's write (Section 2.1)."""
    x = _inputs("gdn", lens=(1,), dk=7, dv=3, h0_std=0.0)
    o, _ = _run(x)
    q, k = x["q"][0, 0].astype(np.float64), x["k"][0, 0].astype(np.float64)
    want = float(x["beta"][0, 0]) * (q @ k) * x["v"][0, 0].astype(np.float64)
    np.testing.assert_allclose(o[0, 0], want, rtol=1e-14)


def test_transition_matrix_form():
    """Brute force on a tiny input with a third algorithm: build each token's
    dk x dk transition M_t = alpha_t (I - beta_t k_t k_t^T) and source
    N_t = beta_t k_t v_t^T explicitly and compose S_t = M_t S_{t-1} + N_t."""
    x = _inputs("gdn", lens=(9,), dk=4, dv=3, h0_std=0.4)
    o, ht = _run(x)
    S = x["h0"][0, 0].astype(np.float64)
    for t in range(9):
        k = x["k"][t, 0].astype(np.float64)
        a = np.exp(float(x["g"][t, 0]))
        b = float(x["beta"][t, 0])
        M = a * (np.eye(4) - b * np.outer(k, k))
        S = M @ S + b * np.outer(k, x["v"][t, 0].astype(np.float64))
        np.testing.assert_allclose(o[t, 0], S.T @ x["q"][t, 0].astype(np.float64), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-13, atol=1e-15)


# ---- the two independent algorithms agree --------------------------------

@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunked_form_equals_recurrence(kind, chunk):
    """The chunkwise Map-Reduce-Map form and the token recurrence are two
    independent algorithms; they must agree to fp64 rounding for any chunk
    size, partial last chunks, dk != dv, grouped heads, varlen and a nonzero
    initial state."""
    x = _inputs(kind, lens=(70, 1, 133), h_qk=2, h_v=4, dk=10, dv=6, h0_std=0.05)
    o1, h1 = _run(x)
    o2, h2 = _run(x, fn=oracle.chunked, chunk=chunk)
    assert _rel(o2, o1) < 1e-12
    assert _rel(h2, h1) < 1e-12


def test_kda_with_uniform_gate_equals_gdn():
    """KDA whose per-channel gate is the same on every channel is GDN."""
    x = _inputs("gdn", lens=(50,), dk=8, dv=6, h0_std=0.1)
    o1, h1 = _run(x)
    xk = dict(x)
    xk["kind"] = "kda"
    xk["g"] = np.repeat(x["g"][:, :, None], 8, axis=2)
    o2, h2 = _run(xk)
    assert _rel(o2, o1) < 1e-13 and _rel(h2, h1) < 1e-13


def test_grouped_heads_use_contiguous_groups():
    """v-head h reads q/k head h // (h_v / h_qk): equal to a call with q/k
    repeated explicitly in that order."""
    x = _inputs("gdn", lens=(40,), h_qk=2, h_v=6, dk=8, dv=4, h0_std=0.1)
    o1, h1 = _run(x)
    xr = dict(x)
    idx = np.arange(6) // 3
    xr["q"] = x["q"][:, idx]
    xr["k"] = x["k"][:, idx]
    o2, h2 = _run(xr)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)
    # and it differs from the interleaved reading h % h_qk
    xi = dict(x)
    xi["q"] = x["q"][:, np.arange(6) % 2]
    xi["k"] = x["k"][:, np.arange(6) % 2]
    o3, _ = _run(xi)
    assert _rel(o3, o1) > 1e-3


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_varlen_equals_separate_calls(kind):
    x = _inputs(kind, lens=(17, 64, 0, 90), h_qk=1, h_v=2, dk=8, dv=4, h0_std=0.1)
    o, ht = _run(x)
    cu = x["cu_seqlens"]
    kda = kind == "kda"
    for s in range(4):
        a, b = cu[s], cu[s + 1]
        o_s, h_s = oracle.recurrence(x["q"][a:b], x["k"][a:b], x["v"][a:b],
                                     x["beta"][a:b], x["g"][a:b],
                                     x["h0"][s:s + 1], kda=kda)
        np.testing.assert_array_equal(o[a:b], o_s)
        np.testing.assert_array_equal(ht[s], h_s[0])
    # a zero-length sequence returns its initial state
    np.testing.assert_array_equal(ht[2], x["h0"][2])


@pytest.mark.parametrize("split", [1, 63, 64, 65, 100])
def test_split_invariance(split):
    """Prefill [0,T) in one call equals [0,t) then [t,T) continued from the
    returned state (the continuation the state hand-off makes possible)."""
    x = _inputs("kda", lens=(150,), dk=8, dv=4, h0_std=0.1)
    o, ht = _run(x)
    kw = dict(kda=True)
    o1, h1 = oracle.recurrence(x["q"][:split], x["k"][:split], x["v"][:split],
                               x["beta"][:split], x["g"][:split], x["h0"], **kw)
    o2, h2 = oracle.recurrence(x["q"][split:], x["k"][split:], x["v"][split:],
                               x["beta"][split:], x["g"][split:], h1, **kw)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), o)
    np.testing.assert_array_equal(h2, ht)


def test_chunked_intermediates_are_consistent():
    """Structure of the chunk intermediates: A strictly lower, T unit lower
    and the inverse of I + A, and V' = U - W h."""
    x = _inputs("gdn", lens=(100,), dk=8, dv=6, h0_std=0.1)
    _, _, inter = oracle.chunked(x["q"], x["k"], x["v"], x["beta"], x["g"],
                                 x["h0"], intermediates=True)
    for it in inter[0]:
        n = it["A"].shape[0]
        assert np.all(np.triu(it["A"]) == 0)
        np.testing.assert_allclose(np.diag(it["T"]), 1.0)
        assert np.all(np.triu(it["T"], 1) == 0)
        np.testing.assert_allclose((np.eye(n) + it["A"]) @ it["T"], np.eye(n), atol=1e-12)
        np.testing.assert_allclose(it["Vp"], it["U"] - it["W"] @ it["h"], atol=1e-12)


# ---- generator -------------------------------------------------------------

def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    # include exact ties
    x[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 3.0], dtype=np.float32)
    ours = W.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_f16_round_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-4, 4, 100000)).astype(np.float32)
    # exact ties between neighbouring halves (1 + 2^-11, 1 + 3 * 2^-11) and a subnormal
    x[:4] = np.array([1.00048828125, 1.00146484375, -1.00048828125, 3e-6], dtype=np.float32)
    ours = W.f16_round(x)
    ref = torch.from_numpy(x).to(torch.float16).float().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_generator_is_deterministic_and_shaped():
    s = W.WORKLOADS["gdn_varlen"]
    assert s.lens == (6745, 1169, 1890, 2330, 1905, 6666, 7188, 4983)
    a = W.make_inputs(W.small_spec("kda", lens=(30, 5), h_qk=2, h_v=4, io="bf16", h0_std=0.02), seed=7)
    b = W.make_inputs(W.small_spec("kda", lens=(30, 5), h_qk=2, h_v=4, io="bf16", h0_std=0.02), seed=7)
    for key in ("q", "k", "v", "beta", "g", "h0"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["g"].shape == (35, 4, 64) and a["h0"].shape == (2, 4, 64, 64)
    np.testing.assert_allclose(np.linalg.norm(a["k"].astype(np.float64), axis=-1), 1.0, atol=1e-2)
    assert np.all(W.bf16_round(a["q"]) == a["q"])
    assert np.all((a["g"] <= -0.01) & (a["g"] >= -0.2))


# ---- decay-only linear attention (RetNet / GLA form, no delta rule) --------

def _decay_parallel_form(q, k, v, g, h0, per_channel):
    """The quadratic ("parallel") form of decay-only linear attention, per
    head, written independently of the token recurrence:
      o_t = (q_t (.) e^{B_t})^T S_0 + sum_{s<=t} sum_d q_td e^{B_td - B_sd} k_sd v_s
      S_T = Diag(e^{B_T}) S_0 + sum_s (k_s (.) e^{B_T - B_s}) v_s^T
    with B the inclusive prefix sum of the log-gates (per key channel, or
    one value broadcast over the channels)."""
    q, k, v, g, h0 = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, h0))
    T, h_v, dk = q.shape[0], v.shape[1], q.shape[2]
    grp = h_v // q.shape[1]
    o = np.zeros_like(v)
    hts = []
    for h in range(h_v):
        qh, kh, vh = q[:, h // grp], k[:, h // grp], v[:, h]
        gh = g[:, h] if per_channel else np.repeat(g[:, h][:, None], dk, axis=1)
        B = np.cumsum(gh, axis=0)                                  # [T, dk]
        S0 = h0[0, h]
        for t in range(T):
            w = np.exp(B[t][None, :] - B[: t + 1])                 # [t+1, dk]
            a = (qh[t][None, :] * w * kh[: t + 1]).sum(axis=1)     # [t+1]
            o[t, h] = (qh[t] * np.exp(B[t])) @ S0 + a @ vh[: t + 1]
        wT = np.exp(B[-1][None, :] - B)
        hts.append(np.exp(B[-1])[:, None] * S0 + (kh * wT).T @ vh)
    return o, np.stack(hts)[None]


@pytest.mark.parametrize("per_channel", [False, True])
def test_decay_only_matches_parallel_form(per_channel):
    """Catches a wrong decay placement (after instead of before the write),
    a dropped initial-state term, or an erase term left in."""
    x = _inputs("kda" if per_channel else "gdn", lens=(23,), h_qk=1, h_v=2, dk=6, dv=4,
                g_lo=0.05, g_hi=0.6)
    o, ht = oracle.recurrence_decay(x["q"], x["k"], x["v"], x["g"], x["h0"],
                                    per_channel=per_channel)
    o_p, ht_p = _decay_parallel_form(x["q"], x["k"], x["v"], x["g"], x["h0"], per_channel)
    assert _rel(o, o_p) < 1e-12 and _rel(ht, ht_p) < 1e-12


def test_decay_only_without_decay_is_causal_linear_attention():
    """g = 0, zero state: O = tril(Q K^T) V, the undecayed causal form."""
    x = _inputs("gdn", lens=(17,), dk=5, dv=3, h0_std=0.0)
    g = np.zeros_like(x["g"])
    o, ht = oracle.recurrence_decay(x["q"], x["k"], x["v"], g, None)
    Q, K, V = x["q"][:, 0].astype(np.float64), x["k"][:, 0].astype(np.float64), x["v"][:, 0]
    assert _rel(o[:, 0], np.tril(Q @ K.T) @ V) < 1e-12
    assert _rel(ht[0, 0], K.T @ V) < 1e-12


def test_decay_only_uniform_channels_equal_scalar_gate():
    x = _inputs("gdn", lens=(30,), h_qk=1, h_v=2, dk=4, dv=4)
    gk = np.repeat(x["g"][:, :, None], 4, axis=2)
    o1, h1 = oracle.recurrence_decay(x["q"], x["k"], x["v"], x["g"], x["h0"])
    o2, h2 = oracle.recurrence_decay(x["q"], x["k"], x["v"], gk, x["h0"], per_channel=True)
    assert _rel(o1, o2) < 1e-13 and _rel(h1, h2) < 1e-13
