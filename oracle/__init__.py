"""FP64 CPU oracle of the Flint sink-aware attention forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""

from .flint_oracle import (  # noqa: F401
    allowed_keys,
    flint_attention,
    kv_head_of,
    rms_norm,
    rope_frequencies,
    rope_neox,
    sink_softmax,
)
from .flint_oracle_bwd import flint_attention_backward  # noqa: F401,E402
from .flint_oracle_bshd import flint_attention_bshd  # noqa: F401,E402
from .flint_oracle_block import flint_attention_block, linear  # noqa: F401,E402
