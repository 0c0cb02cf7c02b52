"""GDN decode with a bf16 state pool, fp64 (oracle; test infrastructure only).

Source: "flashinfer gdn_kernels/gdn_decode_bf16_state.py".

* Gate (``compute_single_gate``): x = a + dt_bias; with softplus parameters
  (beta_sp, threshold) the softplus is log(1 + exp(beta_sp x)) / beta_sp when
  beta_sp x <= threshold and x otherwise; g = -exp(A_log) * softplus;
  alpha = exp(g); beta = 1 / (1 + exp(-b)).
* Normalisation (``normalize_and_store_qk_to_smem``): q_hat = q * scale /
  sqrt(sum q^2 + eps), k_hat = k / sqrt(sum k^2 + eps) over the head dimension,
  eps = 1e-6 (the public ``gated_delta_rule`` entry).  When normalisation is
  off, q_hat = q * scale and k_hat = k.
* Per token, for every (batch b, v-head j) with state slot p = indices[b]:
  S <- alpha S; pred = S k_hat; delta = beta (v - pred); S <- S + delta k_hat^T;
  o = S q_hat.  The state is carried across the T (1..4) tokens of a call and
  written back to the pool as bf16 once, after the last token.
* q/k head of v-head j is j // (HV // H).

Outputs o are returned unrounded (fp64); the new pool is returned with the
updated slots rounded to bf16 and every other slot unchanged.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16
from .recurrence import _f64


def decode_gate(a, b, A_log, dt_bias, softplus_beta: float = 1.0,
                softplus_threshold: float = 20.0):
    """alpha = exp(g) and beta for a, b of shape [..., HV]."""
    a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
    x = a + dt_bias
    bx = softplus_beta * x
    sp = np.where(bx <= softplus_threshold,
                  np.log1p(np.exp(np.minimum(bx, softplus_threshold))) / softplus_beta, x)
    g = -np.exp(A_log) * sp
    return np.exp(g), 1.0 / (1.0 + np.exp(-b))


def decode_normalize(x, eps: float = 1e-6, scale: float = 1.0):
    x = _f64(x)
    return x * (scale / np.sqrt((x * x).sum(-1, keepdims=True) + eps))


def gdn_decode(q, k, v, a, b, A_log, dt_bias, state, indices=None, scale=None,
               softplus_beta: float = 1.0, softplus_threshold: float = 20.0,
               use_qk_l2norm: bool = True, eps: float = 1e-6, batches=None,
               round_state: bool = True):
    """Return (o [B, T, HV, V] fp64, new_state [pool, HV, V, K] bf16 values as fp64).

    ``batches`` restricts the run to some batch rows (others: o = 0, slots
    unchanged) -- used to sample large problems.  ``round_state=False``
    returns the updated slots before their bf16 rounding (exact fp64 state).
    """
    q, k, v, state = _f64(q), _f64(k), _f64(v), _f64(state)
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if scale is None:
        scale = K ** -0.5
    if indices is None:
        idx = np.arange(B)
    else:
        idx = np.asarray(indices.cpu().numpy() if hasattr(indices, "cpu") else indices,
                         dtype=np.int64)
    alpha, beta = decode_gate(a, b, A_log, dt_bias, softplus_beta, softplus_threshold)
    if use_qk_l2norm:
        qh, kh = decode_normalize(q, eps, scale), decode_normalize(k, eps, 1.0)
    else:
        qh, kh = q * scale, k
    head_k = np.arange(HV) // (HV // H)
    o = np.zeros((B, T, HV, V))
    new_state = state.copy()
    rows = range(B) if batches is None else batches
    for bi in rows:
        p = idx[bi]
        S = state[p].copy()                                    # [HV, V, K]
        for t in range(T):
            kt, qt = kh[bi, t, head_k], qh[bi, t, head_k]      # [HV, K]
            S *= alpha[bi, t][:, None, None]
            pred = np.einsum("hvk,hk->hv", S, kt)
            delta = beta[bi, t][:, None] * (v[bi, t] - pred)
            S += delta[:, :, None] * kt[:, None, :]
            o[bi, t] = np.einsum("hvk,hk->hv", S, qt)
        new_state[p] = round_to_bf16(S) if round_state else S
    return o, new_state
