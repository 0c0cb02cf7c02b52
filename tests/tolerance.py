"""Parity bars shared by the GPU tests (reference = the fp64 oracle's value,
never rounded).

* fp32 io:  max |x_gpu - x_ref| <= 1e-4.
* bf16 io:  per element |x_gpu - x_ref| <= 2e-2 * RMS(x_ref) + 2^-8 * |x_ref|,
            and RMS(x_gpu - x_ref) <= 2e-2 * RMS(x_ref).

The 2^-8 |x_ref| term bounds the rounding of a bf16 output itself (half a
bf16 ulp is at most 2^-8 |x|): an exact result stored as bf16 already moves
by that much, so it is not counted as computation error.  The 2e-2 * RMS
part is the bf16 bar applied to everything else.

A value that passes through bf16 storage more than once on its way (a
prefill state handed to the bf16 decode pool and then decoded: ``stores``
= 2) may round to neighbouring bf16 values on the two sides at every store
but the last, a full ulp (2 * 2^-8 |x|) apart; the storage term is then
(2 * stores - 1) * 2^-8 |x_ref|.
"""

import numpy as np
import torch

FP32_ATOL = 1e-4
BF16_REL_RMS = 2e-2
BF16_STORE = 2.0 ** -8


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def check(name, got, ref, io_dtype, mask=None, stores=1):
    """Assert parity; returns a dict of the error figures."""
    g, r = to64(got), to64(ref)
    if mask is not None:
        g, r = g[mask], r[mask]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    if g.size == 0:
        return {}
    d = np.abs(g - r)
    err = float(d.max())
    if io_dtype == torch.float32:
        assert err <= FP32_ATOL, f"{name}: max abs err {err:.3e} > {FP32_ATOL:.1e}"
        return {"max_abs": err}
    rms = float(np.sqrt(np.mean(r * r)))
    bound = BF16_REL_RMS * rms + (2 * stores - 1) * BF16_STORE * np.abs(r)
    worst = int(np.argmax(d - bound))
    rel_rms = float(np.sqrt(np.mean(d * d)) / rms) if rms > 0 else 0.0
    assert np.all(d <= bound), (
        f"{name}: |err| {d.flat[worst]:.3e} > bound {bound.flat[worst]:.3e} at ref {r.flat[worst]:.3e} "
        f"(rms {rms:.3e}, max abs err {err:.3e} = {err / max(rms, 1e-300):.4f} rms)")
    assert rel_rms <= BF16_REL_RMS, f"{name}: rms err {rel_rms:.4f} of rms > {BF16_REL_RMS}"
    return {"max_abs": err, "max_over_rms": err / rms if rms else 0.0, "rel_rms": rel_rms}
