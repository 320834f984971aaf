"""Gated DeltaNet-2 forward pass for AMD Instinct MI355X (gfx950).

Two entry points, both hand-written HIP behind the C ABI in include/gdn2.h:

* ``gdn2_chunk_fwd``      chunkwise WY forward over whole sequences (64-token
                          chunks; varlen via ``cu_seqlens``)
* ``gdn2_recurrent_step`` fused single-token decode step, state updated in place
* ``gdn2_recurrent_fwd``  the fused recurrent form over T tokens per sequence
* ``gdn2_chunk_bwd``      gradients of the chunkwise forward (gate-aware backward)
* ``gdn2_mixer_prologue`` / ``gdn2_mixer_epilogue``: the token mixer around the
  recurrence (convolution, SiLU, L2 norm, gate sigmoids; RMS norm and output gate)
* ``gdn2_chunk_fwd_gates`` / ``gdn2_recurrent_step_gates``: the same with a gate
  layout (``GATES_*`` flags: scalar erase, write or decay gates, tied write gate)

Importing the package does not load the library; the first call does.
"""
from .binding import (  # noqa: F401
    GATES_FULL,
    GATES_GDN,
    GATES_KDA,
    GATES_SCALAR_DECAY,
    GATES_SCALAR_ERASE,
    GATES_SCALAR_WRITE,
    GATES_TIED,
    Gdn2Error,
    gdn2_chunk_bwd,
    gdn2_chunk_bwd_workspace_bytes,
    gdn2_chunk_fwd,
    gdn2_chunk_fwd_gates,
    gdn2_chunk_fwd_workspace_bytes,
    gdn2_mixer_epilogue,
    gdn2_mixer_prologue,
    gdn2_recurrent_fwd,
    gdn2_recurrent_step,
    gdn2_recurrent_step_gates,
    load,
    status_string,
)

__all__ = [
    "GATES_FULL",
    "GATES_GDN",
    "GATES_KDA",
    "GATES_SCALAR_DECAY",
    "GATES_SCALAR_ERASE",
    "GATES_SCALAR_WRITE",
    "GATES_TIED",
    "Gdn2Error",
    "gdn2_chunk_bwd",
    "gdn2_chunk_bwd_workspace_bytes",
    "gdn2_chunk_fwd",
    "gdn2_chunk_fwd_gates",
    "gdn2_chunk_fwd_workspace_bytes",
    "gdn2_mixer_epilogue",
    "gdn2_mixer_prologue",
    "gdn2_recurrent_fwd",
    "gdn2_recurrent_step",
    "gdn2_recurrent_step_gates",
    "load",
    "status_string",
]
