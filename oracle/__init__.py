"""fp64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check in the
package entry file and by the CPU-baseline leg of the benchmark, never by the
library or its binding. It shares no code with the HIP path.
"""
from .paged_attention import (  # noqa: F401
    attend,
    gather_sequence,
    kv_store,
    paged_attn_decode,
    paged_attn_prefill,
)
from .rotary import qknorm_rope_kv_store, rms_norm, rope, rope_angles, rope_kv_store  # noqa: F401
from .fp8_kv import dequantize as fp8_dequantize, kv_store_fp8, paged_attn_decode_fp8, quantize as fp8_quantize  # noqa: F401,E501
