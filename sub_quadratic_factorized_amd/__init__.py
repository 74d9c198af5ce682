"""SQuad-Attention on AMD Instinct MI355X (gfx950).

The operator composes a local softmax pass inside windows of the latent grid
with a global softmax pass across windows at each in-window slot.  Compute runs
in the HIP library libsquad_attn.so (C ABI in include/squad_attn.h); this
package holds the ctypes binding, the in-tree build step and the seeded
synthetic workloads.
"""

from .binding import (  # noqa: F401
    SQUAD_BF16,
    SQUAD_F32,
    SquadError,
    squad_attn_bwd,
    squad_attn_bwd_bytes,
    squad_attn_bwd_flops,
    squad_attn_bwd_workspace_bytes,
    squad_attn_bytes,
    squad_attn_flops,
    squad_attn_bytes_padded,
    squad_attn_flops_padded,
    squad_attn_fwd,
    squad_attn_fwd_padded,
    squad_attn_fwd_reversed,
    squad_attn_global,
    squad_attn_local,
    squad_attn_max_len,
    squad_attn_padded_workspace_bytes,
    squad_status_str,
    squad_window_solve,
)
