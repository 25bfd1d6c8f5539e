"""pkv_paged_attention_varlen_noalloc -- the attention call for callers that
cannot allocate (graph capture, tight serving loops): its work list and
split-KV partials live in the library's static device scratch array.

Through the C ABI, two calls in a row (the second with a smaller batch, so
it runs over the first call's leftovers in the shared array) must match
pkv_paged_attention_varlen -- the same kernels over a workspace the caller
allocates -- bit for bit, and the oracle within the bf16 bar."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import binding, workloads

from gpu_helpers import assert_attention_close, bits_view, device, gpu_prepare, log

pytestmark = pytest.mark.gpu

# a batch with prompt tiles and split decode contexts, then a smaller one
BATCHES = [
    ("big", [1, 1, 300, 1, 2, 1], [4000, 900, 200, 2500, 61, 7000], 32, 8, 128, 256),
    ("small", [1, 40, 1], [700, 10, 95], 32, 8, 128, 64),
]


def _written(wl):
    prep, bt = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=16)
    return prep, bt, kc, vc


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    outs = []
    for k, (name, nst, nct, Hq, Hkv, d, split) in enumerate(BATCHES):
        wl = workloads.build(f"noalloc-{name}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=d, seed=600 + k, device=device(), pool_slack=1.2)
        prep, bt, kc, vc = _written(wl)
        kw = dict(max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, scale=wl.scale,
                  split_tokens=split)
        need = pkv.attention_workspace_bytes(wl.num_reqs, wl.num_tokens, Hq, Hkv, d,
                                             wl.max_query_len, wl.max_seq_len, split)
        assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES
        ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=device())
        ref_out = torch.full_like(wl.q, float("nan"))
        pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                            out=ref_out, workspace=ws, **kw)
        got = torch.full_like(wl.q, float("nan"))
        binding.paged_attention_noalloc(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"],
                                        bt, out=got, **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(got).all(), f"{name}: rows left unwritten"
        assert torch.equal(bits_view(got), bits_view(ref_out)), f"{name}: differs from the " \
            "workspace call"
        okc, ovc = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
        ref_prep = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens,
                                  wl.block_table, 16, wl.num_blocks)
        oracle.kv_write(wl.key.cpu(), wl.value.cpu(), okc, ovc, ref_prep["slot_mapping"], 16)
        ref = oracle.attention(wl.q.cpu(), okc, ovc, ref_prep["query_start_loc"],
                               ref_prep["seq_lens"], wl.block_table, 16, wl.scale)
        assert_attention_close(got, ref, wl.dtype, f"noalloc call {k} ({name})")
        outs.append(got)
        log(f"  call {k} ({name}, {wl.num_tokens} rows, {need} scratch bytes): bit-identical to "
            "the workspace call")
