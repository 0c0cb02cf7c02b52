"""Parity bars shared by the GPU tests (reference = the fp64 oracle's value,
never rounded).  The bar depends on the io dtype of the call and on the
dtype the compared tensor is STORED in:

* fp32 io (any output):    max |x_gpu - x_ref| <= 1e-4.
* bf16 io, stored in fp32 (prefill ht, snapshots, state-scan h / dh):
                           max |x_gpu - x_ref| <= rel * RMS(x_ref), rel = 2e-2
                           unless the caller passes a tighter one, and
                           RMS(x_gpu - x_ref) <= rel * RMS(x_ref).
* bf16 io, stored in bf16 (o, decode state, Aqk, Akk_inv, bf16 states):
                           per element |x_gpu - x_ref| <= rel * RMS(x_ref)
                           + 2^-8 * |x_ref|, and the same RMS condition.

The 2^-8 |x_ref| term bounds the rounding of a bf16 output itself (half a
bf16 ulp is at most 2^-8 |x|): an exact result stored as bf16 already moves
by that much, so it is not counted as computation error.  A tensor stored in
fp32 is never rounded to bf16 and gets no such term.

A value that passes through bf16 storage more than once on its way (a
prefill state handed to the bf16 decode pool and then decoded: ``stores``
= 2) may round to neighbouring bf16 values on the two sides at every store
but the last, a full ulp (2 * 2^-8 |x|) apart; the storage term is then
(2 * stores - 1) * 2^-8 |x_ref|.

Every call records its error figures (see ``RECORDS``); the test session
prints them at its end.
"""

import os

import numpy as np
import torch

FP32_ATOL = 1e-4
BF16_REL_RMS = 2e-2
BF16_STORE = 2.0 ** -8
# The state scans take their bf16 inputs exactly and carry the gated operand
# as a bf16 hi + lo pair with fp32 accumulation: their fp32-stored states are
# held to this tighter bar.
STATE_SCAN_REL = 1e-3

# (test id, tensor name, figures) of every check of this process
RECORDS = []


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _stored_dtype(got, stored):
    if stored is not None:
        return stored
    if isinstance(got, torch.Tensor):
        return got.dtype
    raise TypeError("pass stored= for a tensor that is not a torch tensor")


def check(name, got, ref, io_dtype, mask=None, stores=1, rel=None, stored=None):
    """Assert parity; returns (and records) a dict of the error figures.

    ``stored`` is the dtype the compared output is stored in (default: the
    dtype of ``got``, which must then be a torch tensor)."""
    sd = _stored_dtype(got, stored) if io_dtype != torch.float32 else torch.float32
    g, r = to64(got), to64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    if g.size == 0:
        return {}
    d = np.abs(g - r)
    err = float(d.max())
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    if io_dtype == torch.float32:
        RECORDS.append((test, name, {"max_abs": err, "bar": FP32_ATOL}))
        assert err <= FP32_ATOL, f"{name}: max abs err {err:.3e} > {FP32_ATOL:.1e}"
        return {"max_abs": err}
    rel = BF16_REL_RMS if rel is None else rel
    rms = float(np.sqrt(np.mean(r * r)))
    store_term = (2 * stores - 1) * BF16_STORE if sd == torch.bfloat16 else 0.0
    bound = rel * rms + store_term * np.abs(r)
    worst = int(np.argmax(d - bound))
    rel_rms = float(np.sqrt(np.mean(d * d)) / rms) if rms > 0 else 0.0
    fig = {"max_abs": err, "max_over_rms": err / rms if rms else 0.0, "rel_rms": rel_rms,
           "rel": rel, "store_term": store_term}
    RECORDS.append((test, name, fig))
    assert np.all(d <= bound), (
        f"{name}: |err| {d.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} at ref {r.flat[worst]:.3e} "
        f"(rms {rms:.3e}, max abs err {err:.3e} = {err / max(rms, 1e-300):.4f} rms)")
    assert rel_rms <= rel, f"{name}: rms err {rel_rms:.4f} of rms > {rel}"
    return {k: fig[k] for k in ("max_abs", "max_over_rms", "rel_rms")}
