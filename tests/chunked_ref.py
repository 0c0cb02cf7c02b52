"""An independently written fp64 chunked (WY) form of the gated delta rule.

Used only as a pin for the token-by-token oracle: the two are different
algorithms (per-chunk triangular solves and block products here, a sequential
rank-1 recurrence there) that must agree to rounding.

Within a chunk of n tokens with chunk-local cumulative log-gate G and start
state h = S^T (K x V):

  A[r, s]   = beta_r * sum_c k[r, c] k[s, c] exp(G[r, c] - G[s, c])     (s < r)
  Tm        = (I + A)^-1
  u         = Tm (beta * V)
  w         = Tm (beta * exp(G) * K)
  D         = u - w h                                   (the corrected values)
  o         = scale * [ (Q * exp(G)) h + P D ],  P[r, s] = sum_c q[r, c] k[s, c]
                                                   exp(G[r, c] - G[s, c]), s <= r
  h_next    = diag(exp(G_last)) h + (K * exp(G_last - G))^T D

This is the structure the chunked pages use (beta K K^T + solve_tril for Tm,
recompute_w_u for w and u, ``chunk_fwd_kernel_h`` for the state carry).
"""

from __future__ import annotations

import numpy as np


def chunked_delta_rule(q, k, v, beta, scale, g=None, gk=None, h0=None, chunk=16,
                       cu_seqlens=None, intra=None):
    """Return (o, ht) like the recurrent oracle.

    ``intra`` may hold externally computed (Aqk, Akk_inv) arrays laid out
    [B, T, HV, chunk] (row per token); they then replace P*scale and Tm.
    """
    q, k, v, beta = (np.asarray(x, np.float64) for x in (q, k, v, beta))
    B, T, Hk, K = q.shape
    HV, V = v.shape[2:]
    r = HV // Hk
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, np.int64)
        seqs = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    o = np.zeros((B, T, HV, V))
    ht = np.zeros((len(seqs), HV, V, K))
    for n_i, (b, bos, eos) in enumerate(seqs):
        for j in range(HV):
            jk = j // r
            h = np.zeros((K, V)) if h0 is None else np.asarray(h0, np.float64)[n_i, j].T.copy()
            for c0 in range(bos, eos, chunk):
                c1 = min(c0 + chunk, eos)
                n = c1 - c0
                Q, Km, Vm = q[b, c0:c1, jk], k[b, c0:c1, jk], v[b, c0:c1, j]
                bt = beta[b, c0:c1, j]
                if gk is not None:
                    G = np.cumsum(np.asarray(gk, np.float64)[b, c0:c1, j], axis=0)
                elif g is not None:
                    G = np.cumsum(np.asarray(g, np.float64)[b, c0:c1, j])[:, None] * np.ones((1, K))
                else:
                    G = np.zeros((n, K))
                M = np.zeros((n, n))
                P = np.zeros((n, n))
                for rr in range(n):
                    for ss in range(rr + 1):
                        e = np.exp(G[rr] - G[ss])
                        P[rr, ss] = np.sum(Q[rr] * Km[ss] * e)
                        if ss < rr:
                            M[rr, ss] = bt[rr] * np.sum(Km[rr] * Km[ss] * e)
                if intra is not None:
                    Aqk, Ainv = intra
                    P = np.asarray(Aqk, np.float64)[b, c0:c1, j, :n] / scale
                    Tm = np.asarray(Ainv, np.float64)[b, c0:c1, j, :n]
                else:
                    Tm = np.linalg.solve(np.eye(n) + M, np.eye(n))
                u = Tm @ (bt[:, None] * Vm)
                w = Tm @ (bt[:, None] * np.exp(G) * Km)
                D = u - w @ h
                o[b, c0:c1, j] = scale * ((Q * np.exp(G)) @ h + P @ D)
                Gl = G[-1]
                h = np.exp(Gl)[:, None] * h + (Km * np.exp(Gl[None, :] - G)).T @ D
            ht[n_i, j] = h.T
    return o, ht
