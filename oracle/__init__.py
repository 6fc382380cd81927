"""Float64 CPU checker (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path. See ``oracle.attention`` for what it computes.
"""

from .attention import (CAUSAL, CROSS, EMPTY_SENTINEL, FULL, apply_rope, attention_backward,
                        attention_forward, decode_forward, rope_table, window_length)

__all__ = ["CAUSAL", "FULL", "CROSS", "EMPTY_SENTINEL", "apply_rope", "attention_backward",
           "attention_forward", "decode_forward", "rope_table", "window_length"]
