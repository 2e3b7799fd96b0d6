"""fp64 CPU oracle for the nanochat causal self-attention block forward.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the HIP library computes. Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (the C-ABI library and its Python binding) never
imports, links or calls anything here, and nothing here imports the product.

Parity status of each function is stated in its module docstring:
  * ``rope``: the pairing of dimensions (adjacent pairs) and the rotation sign
    (+p*theta) are readings of the pages, which fix neither:
    parity unpinned for those two conventions (everything else pinned).
  * ``qk_norm``: the epsilon (1e-6) is a reading; parity unpinned for eps.
  * ``attention`` / ``decode`` / ``prefill`` / ``decode_shared`` / ``value_gate``: pinned (see tests/test_oracle_pins.py).
  * ``backward`` (``attn_fwd_lse``, ``rope_bwd``, ``qk_norm_bwd``,
    ``attention_core_bwd``, ``attn_bwd``): pinned by finite differences of the
    forward, closed forms, float64 autograd of the core and the GQA identity.
  * ``projection`` (``qkv_rope_qknorm``): pinned by scalar brute force, the
    identity-weight and zero-weight cases and linearity.
"""
from .reference import (  # noqa: F401
    EPS,
    rope_inv_freq,
    rope,
    qk_norm,
    rope_qknorm,
    band_mask,
    attention_core,
    attn_fwd,
    attn_fwd_rows,
    attn_decode,
    attn_prefill,
    attn_decode_shared,
    value_gate,
)
from .projection import qkv_rope_qknorm  # noqa: F401
from .backward import (  # noqa: F401
    attn_fwd_lse,
    rope_bwd,
    qk_norm_bwd,
    attention_core_bwd,
    attn_bwd,
)
