"""Prefill -> decode state handoff, fp64 values (oracle; test infrastructure only).

Sources: "fla ops/common/chunk_h.py" (``chunk_fwd_kernel_h`` stores the final
state ``ht`` in fp32; with its state-V-first layout a (sequence, head) state is
[V, K], K contiguous) and "flashinfer gdn_kernels/gdn_decode_bf16_state.py"
(the decode reads ``initial_state_source[initial_state_indices[b]]``, a bf16
[pool, HV, V, K] array, and stores back into the same slot).

Handing a prefilled sequence over to decode therefore means: the fp32 state
of sequence n, rounded to bf16 (nearest, ties to even -- the ordinary float
conversion the decode page uses for its own stores), lands in pool slot
indices[n].  Slots no sequence names keep their values; a slot outside
[0, pool) is skipped.
"""

from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16
from .recurrence import _f64


def state_to_pool(ht, pool, indices=None) -> np.ndarray:
    """Return the new pool [pool, HV, V, K] (fp64 values) after writing the
    bf16-rounded states ht [N, HV, V, K] into slots ``indices`` (None: n)."""
    ht = np.asarray(_f64(ht))
    out = np.array(_f64(pool), dtype=np.float64, copy=True)
    N, P = ht.shape[0], out.shape[0]
    if indices is None:
        slots = list(range(N))
    else:
        slots = [int(x) for x in np.asarray(indices.cpu().numpy() if hasattr(indices, "cpu") else indices)]
    for n in range(N):
        p = slots[n]
        if 0 <= p < P:
            out[p] = round_to_bf16(ht[n])
    return out
