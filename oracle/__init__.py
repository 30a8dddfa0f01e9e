"""Plain fp64 CPU oracle for the VGGT Aggregator attention block.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The GPU library never
calls it, links it or falls back to it, and it shares no code, table or helper
with the HIP kernels.
"""

from .vggt_oracle import (  # noqa: F401
    OracleParams,
    frame_attention,
    global_attention,
    register_attention,
    global_attention_rows,
    frame_attention_rows,
    register_attention_rows,
    rope_angles,
    layer_norm_heads,
    rope_2d,
    attention_probs,
    token_positions,
)
from .avggt_sga import (  # noqa: F401
    kept_tokens,
    sga_core,
    sga_attention,
    sga_attention_rows,
)
from .httm import (  # noqa: F401
    HttmParams,
    httm_attention,
    httm_attention_rows,
    fragile,
    merged_length,
)
