"""The bf16 parity bar accepts an exact result stored as bf16 and rejects
planted computation errors (CPU only)."""

import numpy as np
import pytest
import torch

from tests.tolerance import check


def _heavy_tailed(n, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 0.5) * 0.01


def test_exact_result_stored_as_bf16_passes():
    ref = _heavy_tailed(1 << 20, 0)
    stored = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    check("o", stored, ref, torch.bfloat16)


@pytest.mark.parametrize("where", ["outlier", "typical"])
def test_planted_error_fails(where):
    ref = _heavy_tailed(1 << 16, 1)
    got = ref.copy()
    rms = np.sqrt(np.mean(ref ** 2))
    i = int(np.argmax(np.abs(ref))) if where == "outlier" else int(np.argmin(np.abs(np.abs(ref) - rms)))
    got[i] += 0.03 * rms + 2.0 ** -8 * abs(ref[i])
    with pytest.raises(AssertionError):
        check("o", got, ref, torch.bfloat16)


def test_rms_bar_fails_on_uniform_error():
    ref = _heavy_tailed(1 << 16, 2)
    rms = np.sqrt(np.mean(ref ** 2))
    got = ref + 0.019 * rms * np.sign(np.random.default_rng(3).standard_normal(ref.size)) * 1.1
    with pytest.raises(AssertionError):
        check("o", got, ref, torch.bfloat16)


def test_fp32_bar():
    ref = np.linspace(-1, 1, 100)
    check("o", ref + 9e-5, ref, torch.float32)
    with pytest.raises(AssertionError):
        check("o", ref + 1.1e-4, ref, torch.float32)


def test_two_stores_bar():
    """Two paths that store a value as bf16 twice (the second store after a
    factor near 1) may land a full ulp apart at the first store; stores=2
    accepts that and still rejects a planted 3 % * RMS error."""
    rng = np.random.default_rng(4)
    x = _heavy_tailed(1 << 16, 5)
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).double().numpy()
    ref_mid = bf(x)                                  # oracle path: exact value stored once
    ulp = 2.0 ** (np.floor(np.log2(np.abs(ref_mid) + 1e-300)) - 7)
    gpu_mid = ref_mid + ulp * rng.choice([-1.0, 1.0], x.size)   # the other path: one ulp away
    f = 0.97
    ref = ref_mid * f                                # second step, unrounded on the oracle side
    got = bf(gpu_mid * f)                            # ... stored again on the GPU side
    with pytest.raises(AssertionError):
        check("s", got, ref, torch.bfloat16)
    check("s", got, ref, torch.bfloat16, stores=2)
    rms = np.sqrt(np.mean(ref ** 2))
    bad = got.copy()
    i = int(np.argmin(np.abs(np.abs(ref) - rms)))
    bad[i] += 0.03 * rms + 3 * 2.0 ** -8 * abs(ref[i])
    with pytest.raises(AssertionError):
        check("s", bad, ref, torch.bfloat16, stores=2)
