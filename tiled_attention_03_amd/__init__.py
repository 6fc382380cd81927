"""MI355X (gfx950) fused attention forward: prefill and single-token decode
behind a C ABI (include/ta03.h, libta03.so), with a ctypes binding.

The library is loaded lazily on the first call, so importing the package (or
its input generators) needs no GPU and no built library.
"""

from .binding import (CAUSAL, CROSS, FULL, OVERRIDE_BWD_PATH, OVERRIDE_PREFILL_ROWS, Ta03Error,
                      attention, attn_set_kernel_override, attention_backward, attn_bwd,
                      attn_bwd_windows, attn_bwd_workspace_bytes, attn_bwd_workspace_bytes_stored,
                      attn_decode,
                      attn_decode_noalloc, attn_decode_paged, attn_decode_workspace_bytes, attn_decode_workspace_init,
                      attn_fwd, attn_fwd_ex, attn_fwd_rope, attn_fwd_rope_q, attn_rope_apply,
                      attn_rope_table, attn_strerror, lib)

__all__ = ["CAUSAL", "FULL", "CROSS", "OVERRIDE_PREFILL_ROWS", "OVERRIDE_BWD_PATH", "Ta03Error",
           "attn_set_kernel_override", "attention", "attention_backward", "attn_bwd",
           "attn_bwd_windows", "attn_bwd_workspace_bytes", "attn_bwd_workspace_bytes_stored",
           "attn_fwd",
           "attn_fwd_ex",
           "attn_fwd_rope", "attn_fwd_rope_q", "attn_rope_apply", "attn_rope_table", "attn_decode", "attn_decode_noalloc", "attn_decode_paged",
           "attn_decode_workspace_bytes", "attn_decode_workspace_init", "attn_strerror", "lib"]
