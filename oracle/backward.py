"""Backward state-gradient scan, fp64 (oracle; test infrastructure only).

Source: "fla ops/common/chunk_h.py", ``chunk_bwd_kernel_dh``.  Walking the
chunks of a sequence backwards it keeps dh, the gradient with respect to the
state at the end of the current chunk: it starts from dht, stores dh at every
chunk whose index is a multiple of split_size / chunk_size, then applies the
chunk (decay the gradient, add scale * (q o e^G)^T do), and returns dh0 at the
start of the sequence.

Heads: q has Hk heads, dout and the gradients HV, the gates Hg (each a
divisor of HV); v-head j reads q head j // (HV // Hk) and gate head
j // (HV // Hg).  The page's grouped form -- HQ query / output heads whose
programs read the gates of head i_hq // NG, with one dh per query head -- is
Hk = HV = HQ and Hg = HQ // NG.

That is the gradient of the decay-only recurrence
    h_t = D_t h_{t-1} + (terms free of h),   o_t = scale * h_t q_t
(D_t = e^{g_t}, diag(e^{gk_t}) on the key channels and / or diag(e^{gv_t}) on
the value channels, as in the forward state scan), taken token by token
here: at token t (last to first) the output's term scale * do_t q_t^T joins the
gradient of h_t, then the gradient passes to h_{t-1} through D_t.  States are
[V, K] (value rows, key columns), like the forward oracle.
"""

from __future__ import annotations

import numpy as np

from .recurrence import _f64, sequences


def state_grad_scan(q, dout, scale: float, g=None, g_gamma=None, gk=None, gv=None, dht=None,
                    cu_seqlens=None, split_size=None, chunk_size: int = 64):
    """Return (dh [S, HV, V, K] or None, dh0 [N, HV, V, K]), float64.

    dh holds, per sequence (in order), the gradient at the end of chunks
    0, r, 2r, ... (r = split_size / chunk_size): ceil(length / split_size)
    entries per sequence."""
    q, dout = _f64(q), _f64(dout)
    g, gk, gv, dht = _f64(g), _f64(gk), _f64(gv), _f64(dht)
    B, T, Hk, K = q.shape
    HV, V = dout.shape[2], dout.shape[3]
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
    dh0 = np.zeros((len(seqs), HV, V, K))
    snaps = []
    r = None if split_size is None else split_size // chunk_size
    for n, (b, bos, eos) in enumerate(seqs):
        nc = -(-(eos - bos) // chunk_size)
        seq_snaps = [None] * (0 if r is None else -(-(eos - bos) // split_size))
        for j in range(HV):
            kh = j // (HV // Hk)
            jg = j // (HV // Hg)
            D = np.zeros((V, K)) if dht is None else dht[n, j].copy()
            for ic in range(nc - 1, -1, -1):
                if r is not None and ic % r == 0:
                    if seq_snaps[ic // r] is None:
                        seq_snaps[ic // r] = np.zeros((HV, V, K))
                    seq_snaps[ic // r][j] = D
                for t in range(min(bos + (ic + 1) * chunk_size, eos) - 1, bos + ic * chunk_size - 1, -1):
                    D = D + scale * np.outer(dout[b, t, j], q[b, t, kh])
                    if g is not None:
                        D = D * np.exp(g[b, t, jg])
                    if gk is not None:
                        D = D * np.exp(gk[b, t, jg])[None, :]
                    if gv is not None:
                        D = D * np.exp(gv[b, t, jg])[:, None]
            dh0[n, j] = D
        snaps += seq_snaps
    dh = None
    if r is not None:
        dh = np.stack(snaps) if snaps else np.zeros((0, HV, V, K))
    return dh, dh0
