"""MI355X-native KDA (Kimi Delta Attention): gate, chunkwise forward and backward,
decode step, backed by hand-written gfx950 HIP kernels in libkda.so.

Public API (thin wrappers over the C ABI in include/kda.h):
    gate(z, A_log=None, g_min=-5.0, chunk=0, cu_seqlens=None)
    chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
              gate="logdecay", A_log=None, g_min=-5.0, chunk=64, scale=1.0)
    recurrent_step(q, k, v, g, beta, state, gate="logdecay", ...)
    transition(k, g, beta, cu_seqlens=None, gate="logdecay", ...)
    compose_states(M, b, initial_state, nseq, P)
    chunk_fwd_split(q, k, v, g, beta, initial_state=None, cu_seqlens=None, segments=8, ...)
    chunk_fwd_noalloc(q, k, v, g, beta, o, final_state, ...)   (no allocation)
    chunk_fwd_gated(q, k, v, g, beta, out_gate, norm_weight=None, eps=1e-6, ...)
    gated_rmsnorm(o, out_gate, norm_weight=None, eps=1e-6)
    chunk_bwd(q, k, v, g, beta, do, initial_state=None, d_final_state=None, ...)
    gate_bwd(z, dg, A_log=None, g_min=-5.0)
    device_status(clear=False)        (device-side failure flags)
"""
from .ops import (bwd_workspace_size, chunk_bwd, chunk_fwd, chunk_fwd_gated,  # noqa: F401
                  chunk_fwd_noalloc, chunk_fwd_split, chunk_fwd_train, debug_set_spin_limit, device_status, compose_states, gate, gate_bwd, gated_rmsnorm, recurrent_step,
                  transition, workspace_size)

__all__ = ["bwd_workspace_size", "chunk_bwd", "chunk_fwd", "chunk_fwd_gated", "chunk_fwd_noalloc",
           "chunk_fwd_split", "chunk_fwd_train", "debug_set_spin_limit", "device_status",
           "compose_states", "gate", "gate_bwd", "gated_rmsnorm", "recurrent_step",
           "transition", "workspace_size"]
