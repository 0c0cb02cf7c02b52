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
        check("o", got, ref, torch.bfloat16, stored=torch.bfloat16)


def test_rms_bar_fails_on_uniform_error():
    ref = _heavy_tailed(1 << 16, 2)
    rms = np.sqrt(np.mean(ref ** 2))
    got = ref + 0.019 * rms * np.sign(np.random.default_rng(3).standard_normal(ref.size)) * 1.1
    with pytest.raises(AssertionError):
        check("o", got, ref, torch.bfloat16, stored=torch.bfloat16)


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
        check("s", got, ref, torch.bfloat16, stored=torch.bfloat16)
    check("s", got, ref, torch.bfloat16, stores=2, stored=torch.bfloat16)
    rms = np.sqrt(np.mean(ref ** 2))
    bad = got.copy()
    i = int(np.argmin(np.abs(np.abs(ref) - rms)))
    bad[i] += 0.03 * rms + 3 * 2.0 ** -8 * abs(ref[i])
    with pytest.raises(AssertionError):
        check("s", bad, ref, torch.bfloat16, stores=2, stored=torch.bfloat16)


def test_fp32_stored_output_gets_no_storage_term():
    """A tensor stored in fp32 is never rounded to bf16: the bf16 rounding
    of an exact result, passed off as an fp32-stored output, exceeds the
    2e-2 * RMS bar at the tails."""
    ref = _heavy_tailed(1 << 20, 6)
    rounded = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float()
    check("o", rounded.to(torch.bfloat16), ref, torch.bfloat16)       # stored as bf16: passes
    err = np.abs(rounded.double().numpy() - ref)
    assert err.max() > 2e-2 * np.sqrt(np.mean(ref ** 2))                # the premise of the test
    with pytest.raises(AssertionError):
        check("ht", rounded, ref, torch.bfloat16)                        # fp32 tensor: no storage term


def test_state_scan_bar():
    """The state scans' bar (1e-3 * RMS, fp32 storage) accepts fp32 rounding
    noise and rejects a planted 2e-3 * RMS error."""
    from tests.tolerance import STATE_SCAN_REL
    ref = _heavy_tailed(1 << 16, 7)
    got = torch.from_numpy(ref.astype(np.float32))
    check("h", got, ref, torch.bfloat16, rel=STATE_SCAN_REL)
    bad = got.clone()
    bad[17] += 2e-3 * float(np.sqrt(np.mean(ref ** 2)))
    with pytest.raises(AssertionError):
        check("h", bad, ref, torch.bfloat16, rel=STATE_SCAN_REL)


def test_storage_dtype_required_for_numpy():
    ref = _heavy_tailed(64, 8)
    with pytest.raises(TypeError):
        check("o", ref.copy(), ref, torch.bfloat16)
