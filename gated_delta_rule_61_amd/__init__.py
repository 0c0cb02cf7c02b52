"""MI355X (gfx950) gated delta rule: chunked GDN / KDA prefill forward and the
bf16-state decode step, as hand-written HIP kernels behind a C ABI
(``include/gdn61.h``).  The Python entry points below marshal torch tensors
into that ABI; nothing is computed in Python.
"""

from .binding import (GDNError, chunk_bwd_dh, gdn_chunk_fwd, gdn_decode, kda_chunk_fwd, lib,
                      state_to_pool, workspace_bytes)

__all__ = ["GDNError", "chunk_bwd_dh", "gdn_chunk_fwd", "gdn_decode", "kda_chunk_fwd", "lib", "state_to_pool",
           "workspace_bytes"]
__version__ = "0.1.0"
