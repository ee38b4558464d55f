"""FP64 CPU oracle for paged GQA decode attention (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library neither imports nor falls
back to it.
"""

from .decode import (  # noqa: F401
    attend,
    contiguous_decode_attention,
    decode_fp8_e4m3,
    encode_fp8_e4m3,
    gather_sequence,
    lse_merge,
    paged_decode_attention,
    paged_decode_attention_fp8,
    paged_kv_write,
    paged_kv_write_fp8,
    paged_multi_query_attention,
    paged_multi_query_attention_fp8,
    partial_attention,
    quantize_fp8_e4m3,
)
from .prologue import (  # noqa: F401
    attention_prologue,
    attention_prologue_fp8,
    rms_norm_heads,
    rope_angles,
    rope_neox,
    round_bf16,
)
