"""Float64 CPU oracle of the LLaMA decoder layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""
from .layer import (apply_rope, attention_block, causal_gqa_attention, decode_step,  # noqa: F401
                    kv_cache_elements, layer_forward, layer_parameter_count, linear,
                    mlp_block, prefill, project_kv, rms_norm, rope_inv_freq, silu,
                    swiglu_ffn, swiglu_hidden)
from .stack import round_storage, stack_decode_step, stack_prefill  # noqa: F401
