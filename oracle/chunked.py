"""TEST INFRASTRUCTURE ONLY: fp64 chunkwise form of delta-rule prefill.

This follows the Map-Reduce-Map evaluation of "Empowering Hybrid Attention
Models on NPUs", Section 2.1 ("Chunkwise Map-Reduce-Map Execution"), one
chunk at a time in the operator order the page names:

  #1 Gate  -- in-chunk cumulative log-decay b_r = sum_{i<=r} g_i
  #2 KKT   -- A = strict_lower(diag(beta) (K K^T (.) D)), D_ri = e^{b_r-b_i}
  #3 Solve -- T = (I + A)^{-1}
  #4 W/U   -- W = T diag(beta) (e^{b} (.) K),  U = T diag(beta) V
  #5 H     -- V' = U - W S  ("v_c" in Section 5), then
              S <- e^{b_n} S + (e^{b_n - b} (.) K)^T V'
  #6 O     -- O = (e^{b} (.) Q) S + lower_incl(Q K^T (.) D) V'

For KDA the decay is per key channel: the products above carry the
exponent per channel, e.g. A_ri = beta_r sum_c k_rc k_ic e^{b_rc - b_ic},
and the state decays as Diag(e^{b_n}) S.  The page prints none of these
formulas; they are the chunk-level identity that follows from the
token recurrence of Section 2.1 (exact up to rounding; checked against the
recurrence in the pin tests).  Section 5 also names the output's two inputs
(the incoming state and the intermediate v_c), which is the V' above.

Everything is numpy float64; library primitives used: matmul, cumsum, exp
and a dense inverse of a unit lower-triangular matrix.
"""
from __future__ import annotations

import numpy as np


def _chunk(Qc, Kc, Vc, bc, gc, S, kda):
    """One chunk for one head.  Qc,Kc [n,dk]; Vc [n,dv]; bc [n] beta;
    gc [n] or [n,dk]; S [dk,dv] entering state.  Returns (O, S_next, dict)."""
    n = Kc.shape[0]
    # #1 Gate
    B = np.cumsum(gc, axis=0)                     # [n] or [n,dk]
    lower = np.tril(np.ones((n, n), dtype=bool), -1)
    lower_incl = np.tril(np.ones((n, n), dtype=bool), 0)
    if kda:
        # exponent differences per channel, only where i <= r is used
        diff = B[:, None, :] - B[None, :, :]      # [r,i,c]
        diff = np.where(lower_incl[:, :, None], diff, -np.inf)
        E = np.exp(diff)
        KK = np.einsum("rc,ic,ric->ri", Kc, Kc, E)
        QK = np.einsum("rc,ic,ric->ri", Qc, Kc, E)
        eB = np.exp(B)                            # [n,dk]
        Kw = Kc * eB
        Qw = Qc * eB
        Kt = Kc * np.exp(B[-1][None, :] - B)      # e^{b_n - b} (.) K
        gamma = np.exp(B[-1])                     # [dk]
    else:
        D = np.where(lower_incl, np.exp(np.where(lower_incl, B[:, None] - B[None, :], 0.0)), 0.0)
        KK = (Kc @ Kc.T) * D
        QK = (Qc @ Kc.T) * D
        eb = np.exp(B)
        Kw = Kc * eb[:, None]
        Qw = Qc * eb[:, None]
        Kt = Kc * np.exp(B[-1] - B)[:, None]
        gamma = np.exp(B[-1])
    # #2 KKT (strictly lower, beta on the rows)
    A = np.where(lower, bc[:, None] * KK, 0.0)
    # #3 Solve
    T = np.linalg.inv(np.eye(n) + A)
    # #4 W/U
    W = T @ (bc[:, None] * Kw)
    U = T @ (bc[:, None] * Vc)
    # #5 H (read): V' from the incoming state
    Vp = U - W @ S
    # #6 O
    P = np.where(lower_incl, QK, 0.0)
    O = Qw @ S + P @ Vp
    # #5 H (update)
    if kda:
        S_next = gamma[:, None] * S + Kt.T @ Vp
    else:
        S_next = gamma * S + Kt.T @ Vp
    inter = dict(b=B, A=A, T=T, Tb=T * bc[None, :], P=P, Kw=Kw, Qw=Qw, W=W, U=U, Vp=Vp,
                 Kt=Kt, gamma=gamma, h=S.copy())
    return O, S_next, inter


def chunked(q, k, v, beta, g, h0=None, cu_seqlens=None, kda=False,
            chunk: int = 64, intermediates: bool = False):
    """fp64 chunkwise evaluation.  Same layouts and return values as
    ``oracle.recurrence``; with ``intermediates=True`` also returns a list,
    per (sequence, v-head), of per-chunk dicts (b, A, T, Tb = T diag(beta),
    P = lower_incl(Q K^T (.) D), Kw = e^b (.) K, Qw = e^b (.) Q, W, U, Vp,
    Kt, gamma, h = state entering the chunk).  Chunks start at each sequence
    start; the last chunk of a sequence may be shorter."""
    q, k, v, beta, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, beta, g))
    T, h_qk, dk = q.shape
    _, h_v, dv = v.shape
    grp = h_v // h_qk
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    n = len(cu) - 1
    o = np.zeros((T, h_v, dv))
    ht = np.zeros((n, h_v, dk, dv))
    inters = []
    for s in range(n):
        for h in range(h_v):
            hk = h // grp
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[s, h], dtype=np.float64)
            per = []
            for t0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                t1 = min(t0 + chunk, int(cu[s + 1]))
                gc = g[t0:t1, h]
                O, S, it = _chunk(q[t0:t1, hk], k[t0:t1, hk], v[t0:t1, h],
                                  beta[t0:t1, h], gc, S, kda)
                o[t0:t1, h] = O
                per.append(it)
            ht[s, h] = S
            inters.append(per)
    if intermediates:
        return o, ht, inters
    return o, ht
