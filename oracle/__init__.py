"""FP64 CPU oracle for the chunkwise Kimi Delta Attention (KDA) prefill forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its Python
binding) imports, calls or links anything in this package. Only the tests, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP path; the only common module is the seeded input
generator package ``kda_synth``, which holds none of the method's arithmetic.

Sources (cited by page title and section; no source code of any page is copied):

* "FlashKDA column split" (mainlymatmul.com blog), section 1 "FlashKDA in two kernels":
  the per-chunk workspace quantities (K_start, Q_start, K_end, D_{0:15}, A_kk, A_qk) and
  the three chunk equations; section 3.1 for the transposed form.
* "K3's KDA Precision Problem: Why Lower-Bounded Decay Is Necessary", sections
  "How the per-channel decay factor exp(G) enters tile computation" (split-exponent
  form), "Matrix inversion in FlashKDA" (Neumann repeated-squaring inverse) and
  "Numerical experiments on H200" (stress families).
* "flashinfer.kda_prefill" API page: flags, varlen ``cu_seqlens`` contract, the
  ``[N, H, V, K]`` state layout and the state-checkpoint contract.

Modules
-------
``kda_token``   the definition: token-by-token recurrence (pinned, see tests).
``kda_chunk``   the pages' chunk equations and the three inverses of (I + R).
``transforms``  in-kernel q/k L2 norm, beta-from-logit and the lower-bounded gate.
                The gate formula is not printed on the pages: parity unpinned against
                the pages for ``safe_gate`` (only its range and special case are pinned).
"""

from .kda_token import checkpoint_starts, kda_recurrence_fp64, token_step
from .kda_chunk import (
    chunk_quantities,
    chunkwise_forward,
    inverse_explicit,
    inverse_forward_substitution,
    inverse_neumann,
)
from .transforms import l2_normalize, sigmoid, safe_gate

__all__ = [
    "kda_recurrence_fp64",
    "checkpoint_starts",
    "token_step",
    "chunk_quantities",
    "chunkwise_forward",
    "inverse_explicit",
    "inverse_forward_substitution",
    "inverse_neumann",
    "l2_normalize",
    "sigmoid",
    "safe_gate",
]
