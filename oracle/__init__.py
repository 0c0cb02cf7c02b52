"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, fp64 reference that the HIP path is checked
against.  It is imported only by ``tests/``, by ``__graft_entry__.smoke()`` and
by the ``cpu_baseline`` leg of ``bench.py``.  The product path (the C-ABI
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code.

Every function works in float64 on numpy arrays.  Inputs stored in bf16 are
converted exactly, so the oracle sees bit-identical values to the GPU.

Sources (cited by page and function in each module):

* "sglang srt/layers/attention/fla/chunk_fwd.py" -- GDN fused beta*K K^T +
  solve_tril kernel and its host wrapper;
* "fla ops/common/chunk_h.py" -- chunked state recurrence (``chunk_fwd_kernel_h``,
  also as the standalone decay-only state scan) and the backward
  state-gradient scan (``chunk_bwd_kernel_dh``);
* "vLLM kimi_k3 amd ops kda/chunk_intra" -- KDA inter-sub-chunk Aqk/Akk +
  solve_tril fused kernel;
* "flashinfer gdn_kernels/gdn_decode_bf16_state.py" -- GDN decode with a bf16
  state (gate, q/k normalisation, per-token state update) and its state pool,
  into which a prefill's final state is handed over.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (brute-force products of the per-token transition
matrices, an independently written chunked form, closed forms of degenerate
cases, library routines, hand-computed fixtures).  No function is
"parity unpinned".
"""

from .recurrence import delta_rule_recurrent, gdn_recurrent, kda_recurrent
from .intra import chunk_intra_matrices, chunk_intra_wu
from .decode import decode_gate, decode_normalize, gdn_decode
from .bf16 import round_to_bf16
from .handoff import state_to_pool
from .backward import state_grad_scan
from .state_scan import state_scan

__all__ = [
    "delta_rule_recurrent", "gdn_recurrent", "kda_recurrent",
    "chunk_intra_matrices", "chunk_intra_wu",
    "decode_gate", "decode_normalize", "gdn_decode",
    "round_to_bf16", "state_to_pool", "state_grad_scan", "state_scan",
]
