"""Seeded synthetic inputs for the chunked gated-delta-rule forward and the
bf16-state decode step.

This module only draws random numbers and arranges them into the shapes and
dtypes the operators take.  It contains none of the method's arithmetic: no
recurrence, no gate cumsum, no decay, no solve.  The CPU oracle and the HIP
path both receive exactly the tensors produced here (bf16 values are exact in
fp64), so the two sides see bit-identical inputs.

Distributions follow the workload descriptions of the GDN/KDA prefill and
decode problems:

* q, k drawn N(0, 1) and L2-normalised over the head dimension (an input
  property of the prefill workloads; the decode kernel normalises in-kernel
  and so receives raw draws),
* v drawn N(0, 1),
* beta = sigmoid(N(0, 1)),
* GDN log-gate g = -softplus(N(0, 1)) * 0.1 per (token, v-head),
* KDA log-gate gk = -softplus(N(0, 1)) * 0.05 per (token, v-head, channel),
* initial states 0.1 * N(0, 1).

Every array is drawn from ``numpy.random.default_rng(seed)`` in float32 and
then cast (round-to-nearest-even) to the io dtype.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x.astype(np.float64)).astype(np.float32)


def _l2n(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (x64 / np.sqrt((x64 * x64).sum(-1, keepdims=True))).astype(np.float32)


def _to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


@dataclasses.dataclass
class PrefillInputs:
    """One prefill problem.  Tensors live on the CPU; move them with ``.to``."""

    q: torch.Tensor            # [B, T, Hk, K] io dtype
    k: torch.Tensor            # [B, T, Hk, K] io dtype
    v: torch.Tensor            # [B, T, HV, V] io dtype
    beta: torch.Tensor         # [B, T, HV] fp32
    g: Optional[torch.Tensor]  # [B, T, HV] fp32 (GDN) or None
    gk: Optional[torch.Tensor]  # [B, T, HV, K] fp32 (KDA) or None
    h0: Optional[torch.Tensor]  # [N, HV, V, K] fp32 or None
    cu_seqlens: Optional[torch.Tensor]  # [N + 1] int64 or None
    scale: float
    name: str = ""

    @property
    def dims(self):
        B, T, Hk, K = self.q.shape
        HV, V = self.v.shape[2], self.v.shape[3]
        return B, T, Hk, HV, K, V

    @property
    def num_seqs(self) -> int:
        if self.cu_seqlens is None:
            return self.q.shape[0]
        return self.cu_seqlens.numel() - 1

    def tokens(self) -> int:
        B, T = self.q.shape[:2]
        return B * T


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor         # [B, T, H, K] bf16 (raw, normalised in-kernel)
    k: torch.Tensor         # [B, T, H, K] bf16
    v: torch.Tensor         # [B, T, HV, V] bf16
    a: torch.Tensor         # [B, T, HV] bf16
    b: torch.Tensor         # [B, T, HV] bf16
    A_log: torch.Tensor     # [HV] fp32
    dt_bias: torch.Tensor   # [HV] fp32
    state: torch.Tensor     # [pool, HV, V, K] bf16
    indices: Optional[torch.Tensor]  # [B] int32 or None
    scale: float
    name: str = ""


def make_prefill(B: int, T: int, Hk: int, HV: int, K: int, V: int, *,
                 dtype: torch.dtype = torch.bfloat16, seed: int = 0,
                 gate: str = "gdn", g_scale: Optional[float] = None,
                 h0: bool = False, h0_std: float = 0.1,
                 seqlens: Optional[list] = None, scale: Optional[float] = None,
                 normalize_qk: bool = True, name: str = "") -> PrefillInputs:
    """Draw one prefill problem.

    ``gate`` is "gdn" (scalar per-token gate), "kda" (per-channel gate) or
    "none".  ``seqlens`` packs variable-length sequences into B == 1.
    """
    rng = np.random.default_rng(seed)
    if seqlens is not None:
        assert B == 1 and sum(seqlens) == T
    f32 = np.float32
    q = rng.standard_normal((B, T, Hk, K), dtype=f32)
    k = rng.standard_normal((B, T, Hk, K), dtype=f32)
    v = rng.standard_normal((B, T, HV, V), dtype=f32)
    if normalize_qk:
        q, k = _l2n(q), _l2n(k)
    beta = _sigmoid(rng.standard_normal((B, T, HV), dtype=f32))
    g = gk = None
    if gate == "gdn":
        gs = 0.1 if g_scale is None else g_scale
        g = (-_softplus(rng.standard_normal((B, T, HV), dtype=f32)) * gs).astype(f32)
    elif gate == "kda":
        gs = 0.05 if g_scale is None else g_scale
        gk = (-_softplus(rng.standard_normal((B, T, HV, K), dtype=f32)) * gs).astype(f32)
    elif gate != "none":
        raise ValueError(gate)
    N = B if seqlens is None else len(seqlens)
    h0_t = None
    if h0:
        h0_t = torch.from_numpy((rng.standard_normal((N, HV, V, K), dtype=f32) * h0_std).astype(f32))
    cu = None
    if seqlens is not None:
        cu = torch.tensor(np.concatenate([[0], np.cumsum(seqlens)]), dtype=torch.int64)
    return PrefillInputs(
        q=_to(q, dtype), k=_to(k, dtype), v=_to(v, dtype),
        beta=torch.from_numpy(beta),
        g=None if g is None else torch.from_numpy(g),
        gk=None if gk is None else torch.from_numpy(gk),
        h0=h0_t, cu_seqlens=cu,
        scale=float(K ** -0.5) if scale is None else float(scale), name=name)


def draw_seqlens(n: int, lo: int, hi: int, seed: int) -> list:
    """n lengths uniform on the integers [lo, hi] (both ends included)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi, size=n, endpoint=True)]


def make_decode(B: int, T: int, H: int, HV: int, K: int, V: int, *, seed: int = 0,
                pool: Optional[int] = None, indices: Optional[list] = None,
                state_std: float = 0.1, scale: Optional[float] = None,
                name: str = "") -> DecodeInputs:
    rng = np.random.default_rng(seed)
    f32 = np.float32
    bf = torch.bfloat16
    q = rng.standard_normal((B, T, H, K), dtype=f32)
    k = rng.standard_normal((B, T, H, K), dtype=f32)
    v = rng.standard_normal((B, T, HV, V), dtype=f32)
    a = rng.standard_normal((B, T, HV), dtype=f32)
    b = rng.standard_normal((B, T, HV), dtype=f32)
    A_log = rng.standard_normal((HV,), dtype=f32)
    dt_bias = rng.standard_normal((HV,), dtype=f32)
    P = B if pool is None else pool
    state = rng.standard_normal((P, HV, V, K), dtype=f32) * f32(state_std)
    idx = None if indices is None else torch.tensor(indices, dtype=torch.int32)
    return DecodeInputs(q=_to(q, bf), k=_to(k, bf), v=_to(v, bf), a=_to(a, bf), b=_to(b, bf),
                        A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias),
                        state=_to(state, bf), indices=idx,
                        scale=float(K ** -0.5) if scale is None else float(scale), name=name)


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds are 1000 + workload number.
# ---------------------------------------------------------------------------

def gdn_fp32_small(seed: int = 1000) -> PrefillInputs:
    """GDN, fp32 io, B=1 T=256 H=2 K=V=64, zero h0."""
    return make_prefill(1, 256, 2, 2, 64, 64, dtype=torch.float32, seed=seed,
                        gate="gdn", name="gdn_fp32_B1_T256_H2_K64")


def gdn_bf16_b4_t4096(seed: int = 1001) -> PrefillInputs:
    """GDN, bf16 q/k/v, B=4 T=4096 H=16 K=V=128, zero h0, final state stored."""
    return make_prefill(4, 4096, 16, 16, 128, 128, dtype=torch.bfloat16, seed=seed,
                        gate="gdn", name="gdn_bf16_B4_T4096_H16_K128")


def gdn_varlen_gqa(seed: int = 1002) -> PrefillInputs:
    """GDN varlen + GQA: 8 packed sequences of length U[64, 8192], Hk=16, HV=32,
    K=V=128, bf16 io, h0 ~ 0.1 N(0,1)."""
    lens = draw_seqlens(8, 64, 8192, seed)
    return make_prefill(1, sum(lens), 16, 32, 128, 128, dtype=torch.bfloat16, seed=seed,
                        gate="gdn", h0=True, seqlens=lens,
                        name="gdn_varlen8_gqa16x32_K128")


def kda_bf16_b2_t8192(seed: int = 1003) -> PrefillInputs:
    """KDA (per-channel gate), B=2 T=8192 H=32 K=V=128, bf16 io, zero h0."""
    return make_prefill(2, 8192, 32, 32, 128, 128, dtype=torch.bfloat16, seed=seed,
                        gate="kda", name="kda_bf16_B2_T8192_H32_K128")


def decode_b256(T: int = 1, seed: int = 1004) -> DecodeInputs:
    """Decode, bf16 state [256, 32, 128, 128], 16 q/k heads, 32 v heads."""
    return make_decode(256, T, 16, 32, 128, 128, seed=seed + 10 * T,
                       name=f"decode_B256_T{T}_H16_HV32_K128")
