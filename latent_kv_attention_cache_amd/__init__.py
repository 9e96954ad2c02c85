"""Latent-KV chunk attention (VideoMLA hot path) on AMD MI355X.

The compute lives in ``libvmla.so`` (hand-written HIP kernels for gfx950 behind
the C ABI in include/vmla.h); this package is its ctypes binding. Build the
library with ``python -m latent_kv_attention_cache_amd.build``.
"""
from ._binding import (VMLA_OK, VMLA_ERR_NULL, VMLA_ERR_SHAPE, VMLA_ERR_DTYPE, VMLA_ERR_ALIGN,
                       VMLA_ERR_RANGE, VMLA_ERR_WORKSPACE, VMLA_ERR_HIP, VMLA_ERR_OVERLAP, VMLA_F32,
                       VMLA_BF16, EXPORTED, LatentCache, VmlaError, default_dims, load_library, vmla_cache,
                       vmla_dims, vmla_attention_workspace_bytes, vmla_cache_append,
                       vmla_chunk_attention, vmla_latent_attention,
                       vmla_query_prologue, vmla_status_string, vmla_fold_query_weights,
                       vmla_fold_output_weights, vmla_layer_workspace_bytes,
                       vmla_chunk_attention_layer, vmla_layer_query_prologue, vmla_layer_attention,
                       vmla_output_projection, vmla_pack_kv_weights, vmla_explicit_workspace_bytes,
                       vmla_chunk_attention_explicit, vmla_chunk_causal_attention,
                       vmla_chunk_causal_latent_attention, vmla_chunk_causal_attention_explicit,
                       vmla_chunk_attention_noalloc, VMLA_NOALLOC_SCRATCH_BYTES)

__all__ = [
    "VMLA_OK", "VMLA_ERR_NULL", "VMLA_ERR_SHAPE", "VMLA_ERR_DTYPE", "VMLA_ERR_ALIGN",
    "VMLA_ERR_RANGE", "VMLA_ERR_WORKSPACE", "VMLA_ERR_HIP", "VMLA_ERR_OVERLAP", "VMLA_F32",
    "VMLA_BF16", "EXPORTED",
    "LatentCache", "VmlaError", "default_dims", "load_library", "vmla_cache", "vmla_dims",
    "vmla_attention_workspace_bytes", "vmla_cache_append", "vmla_chunk_attention",
    "vmla_query_prologue", "vmla_latent_attention", "vmla_status_string",
    "vmla_fold_query_weights", "vmla_fold_output_weights", "vmla_layer_workspace_bytes",
    "vmla_chunk_attention_layer", "vmla_layer_query_prologue", "vmla_layer_attention",
    "vmla_output_projection", "vmla_pack_kv_weights", "vmla_explicit_workspace_bytes",
    "vmla_chunk_attention_explicit", "vmla_chunk_causal_attention",
    "vmla_chunk_causal_latent_attention", "vmla_chunk_causal_attention_explicit",
    "vmla_chunk_attention_noalloc", "VMLA_NOALLOC_SCRATCH_BYTES",
]
