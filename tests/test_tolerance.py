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
