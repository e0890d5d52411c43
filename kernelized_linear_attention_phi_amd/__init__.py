"""KATA causal forward on MI355X (gfx950): Python front end of libkata.so.

    import kernelized_linear_attention_phi_amd as kata
    o = kata.chunked_fwd(q, k, v, chunk=64)                 # [B,H,T,d_v]
    Sp, zp, S, z = kata.scan_states(k, v, chunk=64)         # per-chunk prefixes
    o1 = kata.decode_step(q1, k1, v1, S, z)                 # one recurrent step
    o2 = kata.flash_fwd(q, k, v)                            # quadratic form (bf16)
    o3 = kata.chunked_fwd(q, k, v, prefix="sequential")     # chunk-by-chunk prefix
    o4 = kata.chunked_fwd(q, k, v, feature="identity")      # first-order feature
    o5 = kata.chunked_fwd_decay(q, k, v, log_decay)         # decay-gated
    kata.chunked_fwd_noalloc_into(q, k, v, o, 64, True)     # no workspace, allocates nothing
    o6 = kata.delta_fwd(q, k, v, beta)                      # DeltaKATA (delta rule)
    o7 = kata.factored_fwd(q, k, v, 2, "multi")             # KATA-Mg / "summed": KATA-Sigma-g

The shared library is loaded on first use; calls raise if it is missing.
"""
from ._binding import (KataError, chunked_fwd, chunked_fwd_into, chunked_fwd_workspace,  # noqa: F401
                       chunked_fwd_decay, chunked_fwd_decay_into, chunked_fwd_decay_workspace,
                       decode_step, decode_step_decay, feature_dim, flash_fwd, lib, phi_dim,
                       scan_states, scan_states_into, chunked_fwd_noalloc_into,
                       NOALLOC_SCRATCH_BYTES, prefix_depth, delta_fwd, delta_fwd_into,
                       decode_step_delta, delta_fwd_workspace, factored_dim, factored_fwd, factored_fwd_into,
                       factored_fwd_workspace, decode_step_factored, LIB_PATH)

__version__ = "0.2.0"
