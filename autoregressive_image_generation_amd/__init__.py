"""Diagonal-aware sparse decode attention on AMD MI355X (gfx950).

Python binding of ``libdsa.so`` (C ABI in ``include/dsa.h``): the functions
carry the C names and only marshal arguments.  Every step of the decode runs
in the HIP kernels; there is no fallback of any kind, and loading fails loudly
when the library has not been built (``python -m
autoregressive_image_generation_amd._build``).
"""
from .binding import (
    DSA_BF16,
    DSA_F32,
    DSA_MXFP8,
    DSA_POLICY_DIAGONAL,
    DSA_POLICY_DIAGONAL_SINK4,
    DSA_POLICY_H2O,
    DSA_POLICY_SLIDING_WINDOW,
    DSA_POLICY_STREAMING_LLM,
    DSA_POLICY_TOVA,
    DSA_PROFILE_STATIC_SCRATCH_BYTES,
    DsaError,
    State,
    dense_append_decode_step,
    dense_append_kv,
    dense_append_prompt,
    dense_decode_step,
    dense_state_init,
    dense_state_workspace_bytes,
    dsa_append_decode_step,
    dsa_append_kv,
    dsa_append_prompt,
    dsa_attention_profile,
    dsa_attention_profile_static,
    dsa_hbm_read_probe,
    dsa_decode_step,
    dsa_last_error,
    dsa_policy_state_init,
    dsa_policy_workspace_bytes,
    dsa_profile_workspace_bytes,
    dsa_read_state,
    dsa_set_stream,
    dsa_set_waves,
    dsa_set_splits,
    dsa_state_destroy,
    dsa_state_init,
    dsa_state_step,
    dsa_state_workspace_bytes,
    dsa_strerror,
    exported_symbols,
    library,
    library_path,
)

__all__ = [name for name in dir() if not name.startswith("_") and name != "binding"]
