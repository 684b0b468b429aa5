"""GDLA oracle (test infrastructure): plain fp64 CPU reference of the method.
Only the tests, the package smoke check and the benchmark's CPU baseline may
import it; the HIP library never does."""

from .gdla_ref import (Cfg, attention_heads, attended_keys, differential_gate_out, gdla_block,
                       gdla_decode, gdla_decode_paged, gdla_layer, gdla_layer_backward, gdla_layer_packed, hybrid_windows,
                       kv_head_of, kv_tokens, latent_expand, latent_expand_from_norm, linear, packed_segments,
                       paged_rows, paged_slot, paged_write, project_tokens, query_tokens, rms_norm, rope,
                       rope_inv_freq, rope_params, sigmoid, yarn_inv_freq, yarn_mscale, attention_heads_backward,
                       rms_norm_backward, rope_backward)

__all__ = ["Cfg", "attention_heads", "attended_keys", "differential_gate_out", "gdla_block",
           "gdla_decode", "gdla_decode_paged", "gdla_layer", "gdla_layer_backward", "gdla_layer_packed", "hybrid_windows",
           "kv_head_of", "kv_tokens", "latent_expand", "latent_expand_from_norm", "linear", "packed_segments",
           "paged_rows", "paged_slot", "paged_write", "project_tokens", "query_tokens", "rms_norm", "rope",
           "rope_inv_freq", "rope_params", "sigmoid", "yarn_inv_freq", "yarn_mscale", "attention_heads_backward",
           "rms_norm_backward", "rope_backward"]
