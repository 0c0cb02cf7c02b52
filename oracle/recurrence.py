"""Token-by-token gated delta rule in fp64 (oracle; test infrastructure only).

The state of one (sequence, v-head) is a V x K matrix S ("V-first": row = value
channel, column = key channel, the layout of the decode state pool in
"flashinfer gdn_kernels/gdn_decode_bf16_state.py", and of
``STATE_V_FIRST`` in "fla ops/common/chunk_h.py").  For every token t, in order,
the decode page's per-token functions apply, in this order:

  decay     S <- exp(g_t) * S                    (GDN, scalar gate per v-head)
            S <- S * diag(exp(gk_t))             (KDA, one gate per key channel)
  predict   pred  = S k_t                        (decay_h..._and_compute_pred)
  delta     delta = beta_t * (v_t - pred)        (v_delta = beta * (v - pred))
  update    S <- S + delta k_t^T                 (update_h_with_delta)
  output    o_t   = scale * S q_t                (compute_output)

which is S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = scale * S_t q_t.  Gates are natural-log values per token (the exp2 forms
of the chunked pages are the same after a log2(e) pre-scale).

Grouped q/k heads: v-head j reads q/k head j // (HV // Hk) (the ``i_h // (H //
Hg)`` head map of the sglang chunk_fwd.py kernel and ``i_hv // (HV // H)`` of
the KDA chunk_intra kernel).

Variable-length batches: with ``cu_seqlens`` (int64, N + 1 entries) the batch
dimension must be 1 and sequence n owns packed tokens
[cu_seqlens[n], cu_seqlens[n+1]) -- the varlen convention of all three chunked
pages.  h0 / ht are indexed by sequence.
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def sequences(B: int, T: int, cu_seqlens) -> list:
    """List of (batch index, first token, end token) per sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = np.asarray(cu_seqlens.cpu().numpy() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                    dtype=np.int64)
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def delta_rule_recurrent(q, k, v, beta, scale: float, g=None, gk=None, h0=None,
                         cu_seqlens=None, heads: Optional[list] = None,
                         split_size: Optional[int] = None):
    """Run the recurrence token by token.

    q, k: [B, T, Hk, K]; v: [B, T, HV, V]; beta: [B, T, HV];
    g: [B, T, HV] or None; gk: [B, T, HV, K] or None; h0: [N, HV, V, K] or None.
    ``heads`` restricts the run to a subset of v-heads (outputs of the other
    heads are left 0) -- used to sample large problems.

    Returns o [B, T, HV, V] and ht [N, HV, V, K], both float64.  With
    ``split_size`` also the state snapshots [S, HV, V, K]: the state before
    token 0, split_size, 2 split_size, ... of every sequence, sequence after
    sequence ("fla ops/common/chunk_h.py", chunk_fwd_kernel_h stores h at the
    chunks whose index is a multiple of split_size / chunk_size, before their
    update; S = sum over sequences of ceil(length / split_size)).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    g, gk, h0 = _f64(g), _f64(gk), _f64(h0)
    B, T, Hk, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if HV % Hk:
        raise ValueError("HV must be a multiple of Hk")
    hs = np.arange(HV) if heads is None else np.asarray(heads, dtype=np.int64)
    kh = hs // (HV // Hk)  # q/k head of each selected v-head
    seqs = sequences(B, T, cu_seqlens)
    o = np.zeros((B, T, HV, V))
    ht = np.zeros((len(seqs), HV, V, K))
    snaps = []
    for n, (b, bos, eos) in enumerate(seqs):
        S = np.zeros((len(hs), V, K)) if h0 is None else h0[n, hs].copy()
        for t in range(bos, eos):
            if split_size is not None and (t - bos) % split_size == 0:
                snap = np.zeros((HV, V, K))
                snap[hs] = S
                snaps.append(snap)
            qt, kt = q[b, t, kh], k[b, t, kh]          # [h, K]
            if g is not None:
                S *= np.exp(g[b, t, hs])[:, None, None]
            if gk is not None:
                S *= np.exp(gk[b, t, hs])[:, None, :]
            pred = np.einsum("hvk,hk->hv", S, kt)
            delta = beta[b, t, hs][:, None] * (v[b, t, hs] - pred)
            S += delta[:, :, None] * kt[:, None, :]
            o[b, t, hs] = scale * np.einsum("hvk,hk->hv", S, qt)
        ht[n, hs] = S
    if split_size is not None:
        return o, ht, (np.stack(snaps) if snaps else np.zeros((0, HV, V, K)))
    return o, ht


def gdn_recurrent(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, heads=None, split_size=None,
                  g_gamma=None):
    """Scalar-gate (GDN) recurrence; ``g`` may be None (no decay).  ``g_gamma``
    [HV] is a fixed per-head log-decay applied at every token, in place of g
    ("fla ops/common/chunk_h.py", USE_G_GAMMA: within a chunk the cumulative
    gate is gamma * (t + 1), i.e. g_t = gamma at each token)."""
    if g_gamma is not None:
        if g is not None:
            raise ValueError("pass g or g_gamma, not both")
        B, T = np.shape(q)[:2]
        g = np.broadcast_to(_f64(g_gamma), (B, T, len(_f64(g_gamma))))
    return delta_rule_recurrent(q, k, v, beta, scale, g=g, h0=h0,
                                cu_seqlens=cu_seqlens, heads=heads, split_size=split_size)


def kda_recurrent(q, k, v, gk, beta, scale, h0=None, cu_seqlens=None, heads=None, split_size=None):
    """Per-channel-gate (KDA) recurrence."""
    return delta_rule_recurrent(q, k, v, beta, scale, gk=gk, h0=h0,
                                cu_seqlens=cu_seqlens, heads=heads, split_size=split_size)
