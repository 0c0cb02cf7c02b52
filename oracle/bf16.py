"""bfloat16 rounding, bit level (oracle; test infrastructure only).

The decode page ("flashinfer gdn_decode_bf16_state.py", ``write_h_chunk_to_smem``
and the final write-back of the state after the last token) stores the fp32
state as bf16 with the ordinary float conversion, i.e. round to nearest, ties
to even.  This is that rounding written on the IEEE bit patterns: the value
is first rounded to float32 (numpy's conversion is round-to-nearest-even),
then the low 16 bits of the float32 pattern are rounded away with ties going
to the even upper half.  NaNs stay NaN.
"""

from __future__ import annotations

import numpy as np


def round_to_bf16(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returns float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(f)
    out = r.view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out
