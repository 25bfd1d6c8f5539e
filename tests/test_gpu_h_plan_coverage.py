"""The attention work list covers every unit of work exactly once.

The plan kernel turns query_start_loc and seq_lens into the list that the
main kernel walks: one item per (request, kv head, prompt tile) for prompt
chunks, then one per (request, kv head, context partition) for decodes
("How vLLM Works Internally: A Deep Dive", "PagedAttention V1/V2": a long
context is cut into partitions whose partial results a second pass merges).
These tests read the list back from the workspace and compare it, as a
multiset, with the units derived here from the batch in plain Python.  The
batches put decode requests whose lengths fall into the same coarse length
rank on both sides of a partition boundary (lengths 256 and 257 at a
256-token partition), the case where ordering decode requests by length
rank alone would drop a partition or duplicate one; batches of more than
1024 requests take the request-order path.  A few of the batches then run
end to end with the output and workspace pre-filled with NaN and are
compared with the oracle.

The list layout read here is the implementation's: a 256-byte header whose
word 0 is the item count and word 4 the count of prompt items at the head of
the list, then one int32 quadruple per item (request, kv head, tile or
partition index, partition count or -1 for a prompt tile).
"""
import collections
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import assert_attention_close, device, log

pytestmark = pytest.mark.gpu

PAIRS_PER_TILE = 16     # MFMA N width: (row, q head) pairs of a decode item
PREFILL_PAIRS = 128     # (row, q head) pairs of a prompt tile


def expected_units(qsl, seq_lens, group, num_kv_heads, split, max_splits):
    """Multiset of (request, kv head, index, count) the list must hold."""
    units = collections.Counter()
    n_pre = 0
    for r in range(len(seq_lens)):
        pairs = int(qsl[r + 1] - qsl[r]) * group
        if pairs > PAIRS_PER_TILE:
            tiles = -(-pairs // PREFILL_PAIRS)
            for k in range(tiles):
                for h in range(num_kv_heads):
                    units[(r, h, k, -1)] += 1
            n_pre += tiles * num_kv_heads
        elif pairs >= 1:
            ns = min(max_splits, max(1, -(-max(int(seq_lens[r]), 1) // split)))
            for k in range(ns):
                for h in range(num_kv_heads):
                    units[(r, h, k, ns)] += 1
    return units, n_pre


def read_list(ws):
    w = ws.cpu()
    head = w[:256].view(torch.int32).numpy()
    n, n_pre = int(head[0]), int(head[4])
    items = w[256:256 + 16 * n].view(torch.int32).numpy().reshape(n, 4)
    return items, n_pre


def plan_and_check(qsl, seq_lens, Hq, Hkv, d, split, what):
    dev = device()
    R = len(seq_lens)
    T = int(qsl[-1])
    max_q = int(np.max(np.diff(qsl))) if R else 0
    max_L = int(np.max(seq_lens)) if R else 0
    need = pkv.attention_workspace_bytes(R, T, Hq, Hkv, d, max_q, max_L, split)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev)
    q_d = torch.from_numpy(np.asarray(qsl, np.int32)).to(dev)
    s_d = torch.from_numpy(np.asarray(seq_lens, np.int32)).to(dev)
    pkv.paged_attention_plan(q_d, s_d, num_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=d, max_query_len=max_q, max_seq_len=max_L,
                             split_tokens=split, workspace=ws)
    torch.cuda.synchronize()
    items, n_pre = read_list(ws)
    max_splits = max(1, -(-max(max_L, 1) // split))
    want, want_pre = expected_units(qsl, seq_lens, Hq // Hkv, Hkv, split, max_splits)
    got = collections.Counter(map(tuple, items.tolist()))
    missing = want - got
    extra = got - want
    assert not missing and not extra, \
        f"{what}: missing {list(missing)[:6]}, extra {list(extra)[:6]}"
    assert n_pre == want_pre, f"{what}: {n_pre} prompt items, expected {want_pre}"
    assert (items[:n_pre, 3] == -1).all() and (items[n_pre:, 3] >= 1).all(), \
        f"{what}: prompt items are not the head of the list"
    return ws


def _bucket(L, top):
    """Length rank of the plan's first ordering: 1024 equal ranges of [0, top]."""
    return (top - min(max(L, 0), top)) * 1023 // top


def test_lengths_256_and_257_at_a_256_token_partition():
    """The advisor's case: contexts 8000, 256 and 257, one token each, 32 q /
    8 kv heads, 256-token partitions.  256 and 257 share a length rank but
    need 1 and 2 partitions."""
    seq = np.array([8000, 256, 257], np.int32)
    assert _bucket(256, 8000) == _bucket(257, 8000)
    qsl = np.array([0, 1, 2, 3], np.int32)
    plan_and_check(qsl, seq, 32, 8, 128, 256, "8000/256/257")
    # end to end, with NaN in the output and the workspace beforehand
    wl = workloads.build("p257", [1, 1, 1], [7999, 255, 256], num_q_heads=32, num_kv_heads=8,
                         head_dim=128, seed=257, device=device(), pool_slack=1.1)
    _run_nan_filled(wl, 256)


def _run_nan_filled(wl, split):
    dev = device()
    from gpu_helpers import gpu_prepare
    prep, bt = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=16)
    need = pkv.attention_workspace_bytes(wl.num_reqs, wl.num_tokens, wl.num_q_heads,
                                         wl.num_kv_heads, wl.head_dim, wl.max_query_len,
                                         wl.max_seq_len, split)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev)
    out = torch.full_like(wl.q, float("nan"))
    pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                        max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                        scale=wl.scale, out=out, split_tokens=split, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), f"{wl.name}: rows left unwritten (NaN)"
    okc, ovc = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
    ref_prep = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                              16, wl.num_blocks)
    oracle.kv_write(wl.key.cpu(), wl.value.cpu(), okc, ovc, ref_prep["slot_mapping"], 16)
    ref = oracle.attention(wl.q.cpu(), okc, ovc, ref_prep["query_start_loc"],
                           ref_prep["seq_lens"], wl.block_table, 16, wl.scale)
    assert_attention_close(out, ref, wl.dtype, f"{wl.name} split {split}")


def _colliding_batch(rng, split):
    """Decode lengths clustered within a few tokens of partition boundaries
    (so that one length rank holds requests with different partition
    counts), a long context that stretches the rank width, and now and then
    short multi-row decodes and prompt chunks."""
    R = int(rng.integers(2, 400))
    top = int(rng.integers(4, 40)) * split + int(rng.integers(0, split))
    kind = rng.random(R)
    q_len = np.ones(R, np.int64)
    q_len[kind < 0.05] = rng.integers(2, 5, int((kind < 0.05).sum()))
    q_len[kind > 0.97] = rng.integers(20, 300, int((kind > 0.97).sum()))
    L = (rng.integers(1, max(2, top // split), R) * split +
         rng.integers(-2, 3, R)).astype(np.int64)
    L[0] = top
    L = np.maximum(L, q_len)
    return q_len, L


@pytest.mark.parametrize("seed", range(4))
def test_random_batches_with_colliding_length_ranks(seed):
    rng = np.random.default_rng(700 + seed)
    collisions = 0
    for trial in range(50):
        split = int(rng.choice([32, 64, 256, 512]))
        Hq, Hkv = [(32, 8), (8, 8), (16, 2), (64, 8), (4, 1)][trial % 5]
        q_len, L = _colliding_batch(rng, split)
        qsl = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
        top = int(L.max())
        b = [_bucket(int(x), top) for x in L]
        ns = [-(-int(x) // split) for x in L]
        by_bucket = collections.defaultdict(set)
        for bb, n, ql in zip(b, ns, q_len):
            if ql * (Hq // Hkv) <= PAIRS_PER_TILE:
                by_bucket[bb].add(n)
        collisions += sum(len(v) > 1 for v in by_bucket.values())
        plan_and_check(qsl, L.astype(np.int32), Hq, Hkv, 128, split,
                       f"seed {seed} trial {trial} (R={len(L)}, split {split})")
    log(f"seed {seed}: {collisions} length ranks held decodes of different partition counts")
    assert collisions > 0


@pytest.mark.parametrize("seed", range(3))
def test_colliding_batches_end_to_end(seed):
    """Small-head batches of the same shape through prepare -> write ->
    attention, NaN-filled output and workspace, against the oracle."""
    rng = np.random.default_rng(900 + seed)
    split = 64
    R = 40
    L = (rng.integers(1, 12, R) * split + rng.integers(-2, 3, R)).astype(np.int64)
    L[0] = 13 * split + 5
    nst = np.ones(R, np.int64)
    nst[rng.random(R) < 0.1] = 3
    nst[1] = 70
    L = np.maximum(L, nst + 1)
    wl = workloads.build(f"collide{seed}", nst.tolist(), (L - nst).tolist(), num_q_heads=8,
                         num_kv_heads=2, head_dim=64, seed=950 + seed, device=device(),
                         pool_slack=1.2)
    _run_nan_filled(wl, split)


def _many_requests(rng, R, split):
    """R requests: mostly single-token decodes of 17..600 tokens, some
    multi-row decodes and a few prompt chunks."""
    q_len = np.ones(R, np.int64)
    kind = rng.random(R)
    q_len[kind < 0.05] = rng.integers(2, 4, int((kind < 0.05).sum()))
    q_len[kind > 0.99] = rng.integers(20, 90, int((kind > 0.99).sum()))
    L = rng.integers(17, 600, R).astype(np.int64)
    on_edge = rng.random(R) < 0.1  # lengths on a partition boundary, or one past it
    L[on_edge] = rng.integers(1, 8, int(on_edge.sum())) * split + rng.integers(0, 2, int(on_edge.sum()))
    L = np.maximum(L, q_len + 1)
    return q_len, L


@pytest.mark.parametrize("R", [1025, 2500])
def test_lists_of_more_requests_than_one_ranking_holds(R):
    """Batches above 1024 requests take the plan's request-order path, 1024
    requests per scan: the list must still hold every unit once."""
    rng = np.random.default_rng(R)
    for split, (Hq, Hkv) in ((64, (8, 2)), (256, (32, 8)), (1024, (4, 4))):
        q_len, L = _many_requests(rng, R, split)
        qsl = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
        plan_and_check(qsl, L.astype(np.int32), Hq, Hkv, 64, split, f"R={R} split {split}")


def test_many_requests_end_to_end():
    """1100 requests through prepare -> write -> attention (request-order
    plan path), NaN-filled output and workspace, against the oracle."""
    rng = np.random.default_rng(1100)
    q_len, L = _many_requests(rng, 1100, 64)
    wl = workloads.build("many_reqs", q_len.tolist(), (L - q_len).tolist(), num_q_heads=8,
                         num_kv_heads=2, head_dim=64, seed=1101, device=device(),
                         pool_slack=1.2)
    _run_nan_filled(wl, 64)
