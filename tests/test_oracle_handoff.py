"""Pins of the oracle's prefill -> decode state handoff (CPU only).

The handoff is a bf16 conversion (nearest, ties to even) scattered into pool
slots, so it reduces to library routines: torch's float32 -> bfloat16 cast and
``index_copy_`` on the CPU.  Rounding ties are planted on purpose."""

import numpy as np
import torch

import oracle


def _states(N, HV, V, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, HV, V, K)).astype(np.float32) * 0.3
    # exact ties: low 16 bits 0x8000 with both parities of the kept part
    u = x.view(np.uint32)
    u[:, :, 0, :8] = (u[:, :, 0, :8] & 0xFFFF0000) | 0x8000
    u[:, :, 1, :8] = (u[:, :, 1, :8] & 0xFFFE0000) | 0x18000
    return x


def test_handoff_matches_torch_cast_and_index_copy():
    N, HV, V, K, P = 5, 3, 16, 8, 9
    ht = _states(N, HV, V, K, 1)
    pool = torch.from_numpy(np.random.default_rng(2).standard_normal((P, HV, V, K)).astype(np.float32)).to(torch.bfloat16)
    idx = [7, 0, 4, 2, 8]
    want = pool.clone().index_copy_(0, torch.tensor(idx), torch.from_numpy(ht).to(torch.bfloat16))
    got = oracle.state_to_pool(ht, pool.float().numpy(), idx)
    assert np.array_equal(got, want.double().numpy())


def test_handoff_identity_and_skipped_slots():
    N, HV, V, K = 4, 2, 8, 8
    ht = _states(N, HV, V, K, 3)
    pool = np.zeros((4, HV, V, K))
    got = oracle.state_to_pool(ht, pool)
    assert np.array_equal(got, torch.from_numpy(ht).to(torch.bfloat16).double().numpy())
    # slots outside [0, pool) are skipped, the other slots keep their values
    pool = np.full((3, HV, V, K), 5.0)
    got = oracle.state_to_pool(ht[:3], pool, [-1, 3, 1])
    assert np.all(got[0] == 5.0) and np.all(got[2] == 5.0)
    assert np.array_equal(got[1], torch.from_numpy(ht[2]).to(torch.bfloat16).double().numpy())


def test_handoff_rounding_is_nearest_even_at_planted_ties():
    ht = _states(1, 1, 4, 8, 4)
    got = oracle.state_to_pool(ht, np.zeros((1, 1, 4, 8)))
    u = ht.view(np.uint32)
    for r in (0, 1):
        for c in range(8):
            hi = int(u[0, 0, r, c]) >> 16
            even = hi + (hi & 1)   # tie: round to the even upper half
            want = np.array([even << 16], dtype=np.uint32).view(np.float32)[0]
            assert got[0, 0, r, c] == want
