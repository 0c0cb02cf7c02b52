"""Per-chunk intra matrices Aqk and (I + Akk)^-1 by definition (oracle).

Sources: "vLLM kimi_k3 amd ops kda/chunk_intra" (``chunk_kda_fwd_kernel_inter_
solve_fused``: off-diagonal Aqk/Akk with per-channel gates, beta row scaling,
``scale`` on Aqk, forward substitution + block merge giving Akk_inv) and
"sglang srt/layers/attention/fla/chunk_fwd.py" (``chunk_gated_delta_rule_fwd_
kkt_solve_kernel``: the same for a scalar gate, strictly lower mask on the
diagonal sub-blocks, result (I + A)^-1 stored row-per-token as [B, T, H, BT]).

Definitions, for a chunk of n <= BT tokens starting at token c0 of its
sequence (chunks start every BT tokens from the sequence start) and the
chunk-local cumulative log-gate G_t = sum_{u = c0..t} g_u (per channel for
KDA; the same value on every channel for GDN):

  Aqk[t, s - c0] = scale * sum_c q[t, c] k[s, c] exp(G[t, c] - G[s, c])   c0 <= s <= t
  Akk[t, s - c0] = beta[t] * sum_c k[t, c] k[s, c] exp(G[t, c] - G[s, c]) c0 <= s <  t
  Akk_inv        = inverse of (I + Akk) over the n x n chunk block

Every other entry of a row (columns >= n, and entries above the diagonal) is
0.  The inverse is taken with ``numpy.linalg.inv``; the pages' forward
substitution on 16 x 16 diagonal blocks followed by the block merge computes the
same matrix up to rounding.  The exponent is formed only on the causal
entries, so the positive differences above the diagonal never reach exp.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .recurrence import _f64, sequences


def chunk_intra_matrices(q, k, beta, scale: float, g=None, gk=None, cu_seqlens=None,
                         chunk_size: int = 64, heads: Optional[list] = None,
                         chunks: Optional[list] = None):
    """Return (Aqk, Akk_inv), each [B, T, HV, chunk_size] float64.

    ``g`` is the per-token GDN gate [B, T, HV], ``gk`` the KDA gate
    [B, T, HV, K]; both are raw per-token log-gates (the cumsum is taken here).
    ``heads`` / ``chunks`` restrict the work to some v-heads / to chunks whose
    global index (over the sequences, in order) is listed.
    """
    q, k, beta, g, gk = _f64(q), _f64(k), _f64(beta), _f64(g), _f64(gk)
    B, T, Hk, K = q.shape
    HV = beta.shape[2]
    BT = chunk_size
    hs = range(HV) if heads is None else heads
    Aqk = np.zeros((B, T, HV, BT))
    Ainv = np.zeros((B, T, HV, BT))
    want = None if chunks is None else set(int(c) for c in chunks)
    ci = -1
    for (b, bos, eos) in sequences(B, T, cu_seqlens):
        for c0 in range(bos, eos, BT):
            ci += 1
            if want is not None and ci not in want:
                continue
            n = min(BT, eos - c0)
            rows = slice(c0, c0 + n)
            causal = np.tril(np.ones((n, n), dtype=bool))
            strict = np.tril(np.ones((n, n), dtype=bool), -1)
            for j in hs:
                jk = j // (HV // Hk)
                qc, kc = q[b, rows, jk], k[b, rows, jk]        # [n, K]
                if gk is not None:
                    G = np.cumsum(gk[b, rows, j], axis=0)       # [n, K]
                elif g is not None:
                    G = np.repeat(np.cumsum(g[b, rows, j])[:, None], K, axis=1)
                else:
                    G = np.zeros((n, K))
                diff = G[:, None, :] - G[None, :, :]            # [t, s, c]
                E = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
                qk = np.einsum("tc,sc,tsc->ts", qc, kc, E)
                kk = np.einsum("tc,sc,tsc->ts", kc, kc, E)
                Aqk[b, rows, j, :n] = scale * np.where(causal, qk, 0.0)
                A = beta[b, rows, j][:, None] * np.where(strict, kk, 0.0)
                Ainv[b, rows, j, :n] = np.linalg.inv(np.eye(n) + A)
    return Aqk, Ainv


def chunk_intra_wu(k, v, beta, g=None, cu_seqlens=None, chunk_size: int = 64, g_cumulative: bool = False,
                   heads: Optional[list] = None):
    """Return (A, w, u) of the scalar-gate intra-chunk step, float64:

      A = (I + Akk)^-1                 [B, T, HV, BT] (rows per token, as above)
      w = A diag(beta e^G) K           [B, T, HV, K]
      u = A diag(beta) V               [B, T, HV, V]

    per chunk and v-head ("sglang srt/layers/attention/fla/chunk_fwd.py",
    chunk_gated_delta_rule_fwd_intra: the fused K K^T + solve, then
    recompute_w_u, which scales the k rows by beta and exp(G) and the v rows
    by beta before the product with A).  ``g`` holds per-token log-gates
    [B, T, HV] (their chunk-local cumulative sums G are taken here) or, with
    ``g_cumulative``, the chunk-local cumulative sums themselves, as that
    page's wrapper takes them; None means no gate.  With w and u, the state
    after a chunk is h_end = e^{G_last} h + (K o e^{G_last - G})^T (u - w h)
    (h = S^T, K x V).
    """
    k, v, beta, g = _f64(k), _f64(v), _f64(beta), _f64(g)
    B, T, Hk, K = k.shape
    HV, V = v.shape[2], v.shape[3]
    BT = chunk_size
    hs = range(HV) if heads is None else heads
    A_out = np.zeros((B, T, HV, BT))
    w_out = np.zeros((B, T, HV, K))
    u_out = np.zeros((B, T, HV, V))
    for (b, bos, eos) in sequences(B, T, cu_seqlens):
        for c0 in range(bos, eos, BT):
            n = min(BT, eos - c0)
            rows = slice(c0, c0 + n)
            strict = np.tril(np.ones((n, n), dtype=bool), -1)
            for j in hs:
                kc = k[b, rows, j // (HV // Hk)]               # [n, K]
                vc = v[b, rows, j]                               # [n, V]
                bc = beta[b, rows, j]                            # [n]
                if g is None:
                    G = np.zeros(n)
                elif g_cumulative:
                    G = g[b, rows, j]
                else:
                    G = np.cumsum(g[b, rows, j])
                E = np.exp(np.where(strict, G[:, None] - G[None, :], 0.0))
                A = bc[:, None] * np.where(strict, (kc @ kc.T) * E, 0.0)
                Ainv = np.linalg.inv(np.eye(n) + A)
                A_out[b, rows, j, :n] = Ainv
                w_out[b, rows, j] = Ainv @ ((bc * np.exp(G))[:, None] * kc)
                u_out[b, rows, j] = Ainv @ (bc[:, None] * vc)
    return A_out, w_out, u_out
