"""Seeded random batches end to end: prepare (alone, or with the work list in
one launch) -> KV write -> attention, against the oracle.

Each case draws a batch shape from the ranges the configurations and the
pages' batches span: 1 to 300 requests, mostly single-token decodes with some
short multi-row decodes and prompt chunks of up to 400 rows, contexts of up to
20000 tokens, sometimes a shared prompt prefix (prefix caching, "How vLLM
Works Internally: A Deep Dive"), head layouts from MHA to GQA with 16 q heads
per kv head, head_dim 64 or 128, bf16, FP8 or fp32 pools, and partition sizes
from 32 tokens to the library's own choice.  The index tensors must equal the
oracle's bit for bit; attention rows (all of them for small batches, a seeded
sample of 64 plus the first and last otherwise) must meet the bar of their
dtype, and every output row must be finite (the output starts as NaN)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import assert_attention_close, device, log

pytestmark = pytest.mark.gpu

HEADS = [(32, 8), (16, 2), (8, 8), (64, 8), (16, 1), (4, 4), (40, 40), (12, 4)]


def _case(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.choice([1, 2, 5, 17, 64, 150, 300]))
    Hq, Hkv = HEADS[rng.integers(len(HEADS))]
    d = int(rng.choice([64, 128]))
    kv = str(rng.choice(["bf16", "bf16", "fp8", "f32"]))
    q_len = np.ones(R, np.int64)
    kind = rng.random(R)
    q_len[kind < 0.15] = rng.integers(2, 5, int((kind < 0.15).sum()))
    q_len[kind > 0.9] = rng.integers(5, 400, int((kind > 0.9).sum()))
    if R <= 2:
        q_len[:] = rng.integers(1, 600, R)
    cap = max(300, 600000 // R)  # keeps the pools (and the oracle's host copies) small
    nct = rng.integers(0, min(cap, int(rng.choice([300, 3000, 20000]))), R).astype(np.int64)
    groups = None
    if R >= 4 and rng.random() < 0.3:
        members = sorted(rng.choice(R, size=int(rng.integers(2, min(R, 6) + 1)),
                                    replace=False).tolist())
        prefix = int(rng.integers(1, 40)) * 16
        nct[members] = np.maximum(nct[members], prefix)
        groups = [(members, prefix)]
    split = int(rng.choice([0, 0, 32, 64, 256, 1024]))
    fused = kv != "f32" and bool(rng.random() < 0.5)
    return rng, R, Hq, Hkv, d, kv, q_len, nct, groups, split, fused


@pytest.mark.parametrize("seed", range(7000, 7040))
def test_random_batch_end_to_end(seed):
    rng, R, Hq, Hkv, d, kv, q_len, nct, groups, split, fused = _case(seed)
    dtype = torch.float32 if kv == "f32" else torch.bfloat16
    what = (f"seed {seed}: R={R} T={int(q_len.sum())} heads {Hq}/{Hkv} d={d} {kv} "
            f"split {split} fused={fused} shared={groups is not None}")
    log(what)
    dev = device()
    wl = workloads.build(f"rand{seed}", q_len.tolist(), nct.tolist(), num_q_heads=Hq,
                         num_kv_heads=Hkv, head_dim=d, dtype=dtype, seed=seed, device=dev,
                         pool_slack=1.2, shared_prefix_groups=groups)
    if kv == "fp8":
        wl = workloads.to_fp8(wl, 0.05, 0.03)
    nst_d = torch.from_numpy(wl.num_scheduled_tokens).to(dev)
    nct_d = torch.from_numpy(wl.num_computed_tokens).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    need = pkv.attention_workspace_bytes(wl.num_reqs, wl.num_tokens, Hq, Hkv, d,
                                         wl.max_query_len, wl.max_seq_len, split, dtype)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev)
    if fused:
        prep, _ = pkv.prepare_inputs_and_plan(
            nst_d, nct_d, bt, num_tokens=wl.num_tokens, block_size=16, num_blocks=wl.num_blocks,
            num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_query_len=wl.max_query_len,
            max_seq_len=wl.max_seq_len, dtype=dtype, split_tokens=split, workspace=ws)
    else:
        prep = pkv.prepare_inputs(nst_d, nct_d, bt, num_tokens=wl.num_tokens, block_size=16,
                                  num_blocks=wl.num_blocks)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    ks = vs = None
    if kv == "fp8":
        ks = torch.tensor([wl.kv_scales[0]], dtype=torch.float32, device=dev)
        vs = torch.tensor([wl.kv_scales[1]], dtype=torch.float32, device=dev)
        pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], ks, vs,
                               block_size=16)
    else:
        pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=16)
    out = torch.full_like(wl.q, float("nan"))
    pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                        max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                        scale=wl.scale, out=out, split_tokens=split, workspace=ws, k_scale=ks,
                        v_scale=vs, planned=fused)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), f"{what}: rows left unwritten"

    ref_prep = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                              16, wl.num_blocks)
    for k in ("req_indices", "positions", "slot_mapping", "query_start_loc", "seq_lens",
              "logits_indices"):
        assert np.array_equal(prep[k].cpu().numpy(), np.asarray(ref_prep[k])), f"{what}: {k}"
    T = wl.num_tokens
    rows = None if T <= 96 else np.unique(np.concatenate([rng.choice(T, 64, replace=False),
                                                          [0, T - 1]]))
    okc, ovc = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
    if kv == "fp8":
        oracle.kv_write_fp8(wl.key.cpu(), wl.value.cpu(), okc, ovc, ref_prep["slot_mapping"], 16,
                            *wl.kv_scales)
    else:
        oracle.kv_write(wl.key.cpu(), wl.value.cpu(), okc, ovc, ref_prep["slot_mapping"], 16)
    ref = oracle.attention(wl.q.cpu(), okc, ovc, ref_prep["query_start_loc"],
                           ref_prep["seq_lens"], wl.block_table, 16, wl.scale, rows=rows,
                           kv_scales=wl.kv_scales)
    got = out.cpu() if rows is None else out.cpu()[torch.from_numpy(rows)]
    assert_attention_close(got, ref, dtype, what)
