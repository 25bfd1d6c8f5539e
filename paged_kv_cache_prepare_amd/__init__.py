"""Paged KV-cache input preparation, KV-cache write and paged varlen attention
for AMD Instinct MI355X (gfx950).

The compute lives in ``libpkv.so`` (HIP kernels behind the C ABI declared in
``include/pkv.h``); :mod:`.binding` marshals torch tensors into those calls.
"""
from .binding import (PkvError, attention_workspace_bytes, copy_blocks, kv_cache_write,
                      kv_cache_write_fp8, load, paged_attention, paged_attention_plan,
                      prepare_input_ids, prepare_inputs, prepare_inputs_and_plan, zero_blocks)

__all__ = ["PkvError", "attention_workspace_bytes", "copy_blocks", "kv_cache_write",
           "kv_cache_write_fp8", "load", "paged_attention", "paged_attention_plan",
           "prepare_input_ids", "prepare_inputs", "prepare_inputs_and_plan", "zero_blocks"]
