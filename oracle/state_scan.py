"""Forward chunk-state scan of the decay-only recurrence, fp64 (oracle; test
infrastructure only).

Source: "fla ops/common/chunk_h.py", ``chunk_fwd_kernel_h`` (the common
state scan, without the delta rule's erase term).  For one (sequence, head)
it walks the chunks in order, stores the state at the start of every chunk
whose index is a multiple of split_size / chunk_size, then applies the
chunk: the state decays by the chunk's total gate and gains
sum_t (k_t o e^{G_last - G_t}) (v_t o e^{Gv_last - Gv_t})^T.

Taken token by token here, that is the recurrence
    S_t = diag(e^{gv_t}) S_{t-1} diag(e^{gk_t}) e^{g_t} + v_t k_t^T
on states S [V, K] (value rows, key columns, like the other oracles): the
scalar gate g (or the fixed per-head g_gamma) scales the whole state, the
per-key-channel gate gk its columns, the per-value-channel gate gv its rows;
any absent gate is 1.  Summed over a chunk it gives the chunk form above
exactly (the chunk-local cumulative gates telescope).
"""

from __future__ import annotations

import numpy as np

from .recurrence import _f64, sequences


def state_scan(k, v, g=None, g_gamma=None, gk=None, gv=None, h0=None, cu_seqlens=None,
               split_size=None, chunk_size: int = 64):
    """Return (h [S, HV, V, K] or None, ht [N, HV, V, K]), float64.

    k [B, T, Hk, K]; v [B, T, HV, V]; g [B, T, Hg]; g_gamma [Hg]; gk [B, T, Hg, K];
    gv [B, T, Hg, V]; h0 [N, HV, V, K]; v-head j reads k head j // (HV // Hk)
    and gate head j // (HV // Hg) (Hg = HV unless the gates have fewer heads).  h holds, per sequence (in order), the
    state at the start of chunks 0, r, 2r, ... (r = split_size / chunk_size):
    ceil(length / split_size) entries per sequence."""
    k, v = _f64(k), _f64(v)
    g, gk, gv, h0 = _f64(g), _f64(gk), _f64(gv), _f64(h0)
    B, T, Hk, K = k.shape
    HV, V = v.shape[2], v.shape[3]
    # gate heads: Hg of them, a divisor of HV; v-head j takes gate head
    # j // (HV // Hg) (the page's grouped form: several query / output heads
    # share the gates of one head)
    if g_gamma is not None:
        gam = _f64(g_gamma)
        g = np.broadcast_to(gam, (B, T, gam.shape[0]))
    heads = {x.shape[2] for x in (g, gk, gv) if x is not None}
    assert len(heads) <= 1, "the gates disagree on their head count"
    Hg = heads.pop() if heads else HV
    assert HV % Hg == 0
    seqs = sequences(B, T, cu_seqlens)
    ht = np.zeros((len(seqs), HV, V, K))
    snaps = []
    r = None if split_size is None else split_size // chunk_size
    for n, (b, bos, eos) in enumerate(seqs):
        nc = -(-(eos - bos) // chunk_size)
        seq_snaps = [None] * (0 if r is None else -(-(eos - bos) // split_size))
        for j in range(HV):
            kh = j // (HV // Hk)
            jg = j // (HV // Hg)
            S = np.zeros((V, K)) if h0 is None else h0[n, j].copy()
            for ic in range(nc):
                if r is not None and ic % r == 0:
                    if seq_snaps[ic // r] is None:
                        seq_snaps[ic // r] = np.zeros((HV, V, K))
                    seq_snaps[ic // r][j] = S
                for t in range(bos + ic * chunk_size, min(bos + (ic + 1) * chunk_size, eos)):
                    if g is not None:
                        S = S * np.exp(g[b, t, jg])
                    if gk is not None:
                        S = S * np.exp(gk[b, t, jg])[None, :]
                    if gv is not None:
                        S = S * np.exp(gv[b, t, jg])[:, None]
                    S = S + np.outer(v[b, t, j], k[b, t, kh])
            ht[n, j] = S
        snaps += seq_snaps
    h = None
    if r is not None:
        h = np.stack(snaps) if snaps else np.zeros((0, HV, V, K))
    return h, ht
