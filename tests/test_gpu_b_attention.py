"""GPU parity of pkv_paged_attention_varlen against the fp64 oracle, through
the C ABI: the five named configurations at full size (in the launch
configuration the benchmark times; every output row must be written, every
decode row and a row of every prompt tile is compared), and small cases that span several
tiles with ragged tails, every GQA group size, both head sizes and dtypes,
forced context partitions, NaN-poisoned pools and bad block ids."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import (assert_attention_close, assert_prepare_equal, bits_view, device,
                         gpu_step, log, oracle_step)

pytestmark = pytest.mark.gpu


PAIRS_PER_TILE = 16    # (row, q head) columns of a decode item
PREFILL_PAIRS = 128    # (row, q head) pairs of one prompt tile of one kv head


def sample_rows(wl, seed=0, small=64):
    """Rows the full-size checks compare with the oracle: every row of a
    decode request (q_len * G <= 16), and for each prompt chunk its first and
    last rows plus one seeded random row from every 128-pair tile.  A row
    covers all q heads, so every (kv head, row tile) item of the launch holds
    a compared row.  Returns None (all rows) for batches of at most ``small``
    rows; otherwise the rows, with the prompt tiles covered asserted equal to
    the tiles launched."""
    T = wl.num_tokens
    if T <= small:
        return None
    G = wl.num_q_heads // wl.num_kv_heads
    rng = np.random.default_rng(seed)
    qsl = np.concatenate([[0], np.cumsum(wl.num_scheduled_tokens)]).astype(np.int64)
    rows = set()
    tiles_launched = tiles_covered = 0
    for r in range(wl.num_reqs):
        n = int(wl.num_scheduled_tokens[r])
        if n == 0:
            continue
        if n * G <= PAIRS_PER_TILE:
            rows.update(range(int(qsl[r]), int(qsl[r + 1])))
            continue
        rows.update((int(qsl[r]), int(qsl[r + 1]) - 1))
        n_tiles = -(-n * G // PREFILL_PAIRS)
        tiles_launched += n_tiles
        for t in range(n_tiles):
            lo = PREFILL_PAIRS * t // G
            hi = min(n - 1, (PREFILL_PAIRS * t + PREFILL_PAIRS - 1) // G)
            rows.add(int(qsl[r]) + int(rng.integers(lo, hi + 1)))
            tiles_covered += 1
    assert tiles_covered == tiles_launched
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_attention_config(idx):
    log(f"config {idx}: {workloads.CONFIG_NAMES[idx]}")
    wl = workloads.config(idx, device=device())
    prep, kc, vc, out = gpu_step(wl)
    rows = sample_rows(wl)
    ref_prep, okc, ovc, ref = oracle_step(wl, rows=rows)
    assert_prepare_equal(prep, ref_prep, f"config {idx}")
    assert torch.equal(bits_view(kc.cpu()), bits_view(okc)), "K pool"
    assert torch.equal(bits_view(vc.cpu()), bits_view(ovc)), "V pool"
    got = out if rows is None else out[torch.from_numpy(rows).long().to(out.device)]
    assert_attention_close(got, ref, wl.dtype, f"config {idx} ({'all' if rows is None else len(rows)} rows)")


@pytest.mark.parametrize("idx,rows", [(4, "prefill"), (5, "prefill"), (4, "decode")])
def test_attention_config_rows(idx, rows):
    """The prompt rows alone (1256 and 1024 tiles: the resident prefill
    workgroups walk several rounds of the tile list, two per CU) and the
    decode rows alone, as the benchmark's --rows runs time them."""
    wl = workloads.config(idx, device=device())
    group = wl.num_q_heads // wl.num_kv_heads
    short = wl.num_scheduled_tokens * group <= 16
    wl = workloads.select(wl, np.nonzero(short if rows == "decode" else ~short)[0])
    log(f"config {idx} {rows} rows: {wl.num_reqs} requests, {wl.num_tokens} tokens")
    prep, kc, vc, out = gpu_step(wl)
    sel = sample_rows(wl)
    _, _, _, ref = oracle_step(wl, rows=sel)
    got = out if sel is None else out[torch.from_numpy(sel).long().to(out.device)]
    assert_attention_close(got, ref, wl.dtype, f"config {idx} {rows} rows")


# (nst, nct, Hq, Hkv, d) -- decode items, multi-row decode items (q_len * G <= 16),
# prefill tiles with ragged tails, chunks that start mid-sequence, empty requests.
SMALL = [
    ([1, 1, 1, 1], [0, 15, 16, 300], 4, 4, 128),
    ([1] * 9, [5, 31, 32, 33, 63, 64, 100, 511, 1000], 32, 8, 128),
    ([2, 4, 1, 3], [17, 40, 0, 2], 8, 2, 128),             # 2*4, 4*4... multi-row decodes (G=4)
    ([16, 5], [3, 70], 1, 1, 128),                          # G=1, 16 rows still one decode item
    ([300, 1, 0, 47], [0, 90, 12, 200], 8, 2, 128),        # prefill tiles + ragged tail
    ([700], [1234], 32, 8, 128),                            # long chunk mid-sequence
    ([65, 1, 129], [0, 33, 500], 16, 1, 128),               # G=16 (MQA-like)
    ([1, 1, 40], [7, 200, 9], 4, 2, 64),                    # head_dim 64
    ([3, 1], [0, 77], 2, 2, 64),
    ([0, 0, 5, 0], [0, 4, 60, 3], 6, 3, 128),               # G=2 with empty requests
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_attention_small(case, dtype):
    nst, nct, Hq, Hkv, d = SMALL[case]
    wl = workloads.build(f"small{case}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                         dtype=dtype, seed=50 + case, device=device(), pool_slack=1.3,
                         extra_table_cols=2)
    prep, kc, vc, out = gpu_step(wl)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, dtype, f"small{case} {dtype}")


@pytest.mark.parametrize("split_tokens", [32, 64, 96, 256])
def test_attention_forced_partitions(split_tokens):
    """Split-KV (two-pass) results agree with the oracle and with one pass."""
    nst = [1, 1, 1, 2, 1]
    nct = [2000, 31, 700, 901, 129]
    wl = workloads.build("split", nst, nct, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         seed=77, device=device(), pool_slack=1.1)
    _, _, _, one = gpu_step(wl, split_tokens=2048 + 32)
    _, _, _, many = gpu_step(wl, split_tokens=split_tokens)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(one, ref, wl.dtype, "single pass")
    assert_attention_close(many, ref, wl.dtype, f"split {split_tokens}")


def test_attention_automatic_partitions_of_uneven_contexts():
    """The library's own partition size on a batch with fewer (request, kv
    head) items than CUs: contexts of very different lengths get different
    partition counts (here 1, 2 and 11 at the 3776-token size a 256-CU GPU
    picks), and the rows match the oracle; so does the same batch with FP8
    pools."""
    nst = [1, 1, 1]
    nct = [99, 4999, 39999]
    wl = workloads.build("autosplit", nst, nct, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         seed=78, device=device(), pool_slack=1.1)
    need0 = pkv.attention_workspace_bytes(3, 3, 32, 8, 128, 1, 40000, 0, wl.dtype)
    need1 = pkv.attention_workspace_bytes(3, 3, 32, 8, 128, 1, 40000, 40000 // 32 * 32 + 32,
                                          wl.dtype)
    assert need0 > need1, "the automatic choice partitions this batch"
    _, _, _, out = gpu_step(wl)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, wl.dtype, "automatic partitions")
    f8 = workloads.to_fp8(wl, 0.0125, 0.0125)
    _, _, _, out8 = gpu_step(f8)
    _, _, _, ref8 = oracle_step(f8)
    assert_attention_close(out8, ref8, wl.dtype, "automatic partitions, FP8 pools")


def test_attention_many_requests():
    """More requests than the work-list builder ranks at once (1024): the list
    is built chunk by chunk in request order and must still cover every row."""
    rng = np.random.default_rng(11)
    R = 1500
    nst = np.where(rng.random(R) < 0.9, 1, rng.integers(2, 9, R)).astype(np.int32)
    nct = rng.integers(0, 200, R).astype(np.int32)
    wl = workloads.build("many", nst, nct, num_q_heads=8, num_kv_heads=2, head_dim=64, seed=12,
                         device=device())
    _, _, _, out = gpu_step(wl)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, wl.dtype, f"{R} requests")


def test_attention_partitions_beyond_ordered_plan():
    """More partitions per context (2063) than the work list orders partition-major
    (2048): the request-order path runs and the reduce combines them all."""
    wl = workloads.build("longsplit", [1, 1, 3], [66000, 40000, 10], num_q_heads=4,
                         num_kv_heads=1, head_dim=64, seed=13, device=device())
    _, _, _, out = gpu_step(wl, split_tokens=32)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, wl.dtype, "2063 partitions")


def test_attention_several_prompts_and_partitions():
    """Several prompt chunks of different lengths next to decodes with different
    partition counts, so the longest-first ordering reorders requests."""
    nst = [1, 200, 1, 37, 1, 500, 1]
    nct = [90, 10, 3000, 0, 700, 2500, 1500]
    wl = workloads.build("order", nst, nct, num_q_heads=16, num_kv_heads=4, head_dim=128,
                         seed=14, device=device(), pool_slack=1.2)
    _, _, _, ref = oracle_step(wl)
    for st in (0, 256):
        _, _, _, out = gpu_step(wl, split_tokens=st)
        assert_attention_close(out, ref, wl.dtype, f"ordering, split {st}")


def test_attention_block_permutation_invariance():
    """Moving physical blocks (and rewriting the table) leaves the GPU result
    bit-identical: the kernel's arithmetic order depends only on logical order."""
    wl = workloads.build("perm", [1, 40, 1], [300, 20, 1000], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seed=5, device=device(), pool_slack=1.5)
    _, kc, vc, out = gpu_step(wl)
    perm = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(1))
    kc2 = torch.empty_like(kc)
    vc2 = torch.empty_like(vc)
    pd = perm.to(kc.device)
    kc2[pd] = kc
    vc2[pd] = vc
    bt2 = np.where(wl.block_table >= 0, perm.numpy()[np.maximum(wl.block_table, 0)],
                   -1).astype(np.int32)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(wl.num_scheduled_tokens)]),
                       dtype=torch.int32, device=kc.device)
    sl = torch.tensor(wl.num_scheduled_tokens + wl.num_computed_tokens, dtype=torch.int32,
                      device=kc.device)
    out2 = pkv.paged_attention(wl.q, kc2, vc2, qsl, sl, torch.from_numpy(bt2).to(kc.device),
                               max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                               scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(bits_view(out), bits_view(out2))


def test_attention_bad_block_ids_contribute_nothing():
    """A table entry outside the pool contributes no keys and nothing is read
    outside the pool.  For a single-token query every key is visible, so the
    expected result is attention over the table with that entry removed."""
    wl = workloads.build("badid", [1, 1], [100, 100], num_q_heads=4, num_kv_heads=2,
                         head_dim=128, seed=9, device=device())
    dev = device()
    bt = wl.block_table.copy()
    bt[0, 2] = wl.num_blocks + 1000
    bt[1, 0] = -7
    qsl = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    # history only (no write this step): positions 0..99 hold values
    sl = torch.tensor([100, 100], dtype=torch.int32, device=dev)
    out = pkv.paged_attention(wl.q, wl.key_cache, wl.value_cache, qsl, sl,
                              torch.from_numpy(bt).to(dev), max_query_len=1, max_seq_len=100,
                              scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    dropped = np.full_like(bt, -1)
    dropped[0, :6] = np.delete(wl.block_table[0], 2)[:6]
    dropped[1, :6] = np.delete(wl.block_table[1], 0)[:6]
    ref = oracle.attention(wl.q.cpu(), wl.key_cache.cpu(), wl.value_cache.cpu(), [0, 1, 2],
                           [84, 84], dropped, 16, wl.scale)
    assert_attention_close(out, ref, wl.dtype, "bad block ids")


def test_attention_strided_q_and_out():
    """q as a view of a fused projection, out written into a wider buffer."""
    wl = workloads.build("strided", [5, 1, 1], [10, 50, 0], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seed=11, device=device())
    dev = device()
    T = wl.num_tokens
    _, kc, vc, ref_out = gpu_step(wl)
    fused = torch.zeros(T, (8 + 4) * 128, dtype=wl.dtype, device=dev)
    fused[:, :8 * 128] = wl.q.reshape(T, -1)
    qv = fused[:, :8 * 128].view(T, 8, 128)
    big = torch.full((T, 10 * 128), 7.0, dtype=wl.dtype, device=dev)
    ov = big[:, 128:9 * 128].view(T, 8, 128)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(wl.num_scheduled_tokens)]),
                       dtype=torch.int32, device=dev)
    sl = torch.tensor(wl.num_scheduled_tokens + wl.num_computed_tokens, dtype=torch.int32,
                      device=dev)
    pkv.paged_attention(qv, kc, vc, qsl, sl, torch.from_numpy(wl.block_table).to(dev),
                        max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                        scale=wl.scale, out=ov)
    torch.cuda.synchronize()
    assert torch.equal(bits_view(ov.contiguous()), bits_view(ref_out))
    assert (big[:, :128] == 7).all() and (big[:, 9 * 128:] == 7).all()


# Shared-prefix groups: single-token decodes whose first logical blocks are the
# same physical blocks are computed together over the partitions they share.
# (Hq, Hkv, d, nst, nct, groups [(members, prefix tokens)], split_tokens)
SHARED = [
    # G=8: a group of 5 (an item of 4 + a lone member), a group of 2 with a
    # prefix that ends inside a partition, unshared decodes, a prompt chunk and
    # a two-row decode that shares blocks but is not grouped
    (32, 4, 128, [1, 1, 1, 1, 1, 1, 1, 40, 1, 2],
     [1500, 2000, 1100, 3000, 1030, 700, 900, 1200, 520, 1400],
     [([0, 1, 2, 3, 4, 9], 1024), ([6, 8], 496)], (64, 256, 0)),
    # G=1: 40 members, items of 32 + 8
    (8, 8, 128, [1] * 44, [300 + 7 * i for i in range(44)],
     [(list(range(40)), 256)], (64, 0)),
    # G=16 (one kv head), head_dim 64: items of 2 + 1
    (16, 1, 64, [1, 1, 1, 1], [800, 650, 1200, 90], [([0, 1, 2], 512)], (32, 128)),
    # G=4, head_dim 64, two groups side by side
    (16, 4, 64, [1] * 7, [400, 410, 420, 430, 600, 610, 50],
     [([0, 1, 2, 3], 384), ([4, 5], 592)], (96, 0)),
]


@pytest.mark.parametrize("case", range(len(SHARED)))
def test_attention_shared_prefix_groups(case):
    Hq, Hkv, d, nst, nct, groups, splits = SHARED[case]
    wl = workloads.build(f"shared{case}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                         seed=90 + case, device=device(), pool_slack=1.2,
                         shared_prefix_groups=groups)
    _, _, _, ref = oracle_step(wl)
    for st in splits:
        _, _, _, out = gpu_step(wl, split_tokens=st)
        assert_attention_close(out, ref, wl.dtype, f"shared{case} split {st}")


def test_attention_prefix_that_diverges_and_rejoins():
    """Two decodes whose tables agree on blocks 0-5 and 7 but not 6: only the
    partitions before block 6 may be computed once for both."""
    wl = workloads.build("diverge", [1, 1, 1], [700, 650, 300], num_q_heads=16, num_kv_heads=2,
                         head_dim=128, seed=31, device=device(), pool_slack=1.0)
    wl.block_table[1, :6] = wl.block_table[0, :6]
    wl.block_table[1, 7] = wl.block_table[0, 7]
    _, _, _, ref = oracle_step(wl)
    for st in (32, 64, 128):
        _, _, _, out = gpu_step(wl, split_tokens=st)
        assert_attention_close(out, ref, wl.dtype, f"diverging prefix, split {st}")


@pytest.mark.parametrize("Hq,Hkv,d", [(16, 2, 128), (16, 4, 64)])
def test_attention_shared_prefix_beside_prompt_tiles(Hq, Hkv, d):
    """Split decode contexts with shared prefixes in a launch that also holds
    prompt tiles: partitions whose first block another request holds at the
    same position take the shared-prefix load path.  Request 5 shares only
    block 0 with request 0, so its first partition starts on a shared block
    and then diverges."""
    nst = [1] * 6 + [40]
    nct = [900, 950, 1000, 700, 640, 300, 64]
    wl = workloads.build(f"shared_mixed_{d}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=d, seed=57, device=device(), pool_slack=1.2,
                         shared_prefix_groups=[([0, 1, 2], 512), ([3, 4], 256)])
    wl.block_table[5, 0] = wl.block_table[0, 0]
    _, _, _, ref = oracle_step(wl)
    for st in (0, 64, 256):
        _, _, _, out = gpu_step(wl, split_tokens=st)
        assert_attention_close(out, ref, wl.dtype, f"shared prefix beside prompt, split {st}")


# Shared prefixes among split decode contexts of equal length, where every
# sharer's partitions have the same bounds:
#  * requests 0-3: four sharers over two whole partitions (prefix 2048 tokens);
#  * requests 4, 5: two sharers, one with two query rows, whose prefix (704
#    tokens) ends inside the first partition;
#  * requests 6-8: three sharers of one partition;
#  * request 9 shares request 0's blocks with a different length;
#  * requests 10, 11: unshared.
GROUP_NST = [1, 1, 1, 1, 1, 2, 1, 1, 1, 1, 1, 1]
GROUP_NCT = [2999, 2999, 2999, 2999, 1999, 1998, 1499, 1499, 1499, 2899, 2499, 700]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("prompt", [False, True])
def test_attention_equal_length_sharers(kv, prompt):
    nst, nct = list(GROUP_NST), list(GROUP_NCT)
    if prompt:  # a prompt chunk in the same launch
        nst.append(40)
        nct.append(64)
    wl = workloads.build(f"groups_{kv}_{prompt}", nst, nct, num_q_heads=32, num_kv_heads=8,
                         head_dim=128, seed=61, device=device(), pool_slack=1.2,
                         shared_prefix_groups=[([0, 1, 2, 3, 9], 2048), ([4, 5], 704),
                                               ([6, 7, 8], 1024)])
    if kv == "fp8":
        wl = workloads.to_fp8(wl, 0.05, 0.03)
    _, _, _, ref = oracle_step(wl)
    # 0: the library's partitions (about one item per CU); 1024: the same by
    # hand; 64: many short partitions
    for st in (0, 1024, 64):
        _, _, _, out = gpu_step(wl, split_tokens=st)
        assert_attention_close(out, ref, wl.dtype, f"equal-length sharers {kv} prompt={prompt} split {st}")


def _shape_scores(wl, growth, seed):
    """Give every key of kv head h the direction u_h scaled by growth[r](pos),
    plus noise, and every query of that head's group u_h plus noise, so that a
    row's scores follow growth[r] along the key axis.  Steep growth makes the
    running maximum jump by far more than the kernels' lazy-rescale bound
    within one step of keys, so every rescale path runs."""
    g = torch.Generator().manual_seed(seed)
    H, d, G = wl.num_kv_heads, wl.head_dim, wl.num_q_heads // wl.num_kv_heads
    u = torch.where(torch.rand(H, d, generator=g) < 0.5, -1.0, 1.0)
    kc = workloads.key_logical(wl.key_cache.float().cpu(), d, 16)
    for r, f in enumerate(growth):
        for p in range(int(wl.num_computed_tokens[r])):
            b, off = int(wl.block_table[r, p // 16]), p % 16
            kc[b, :, off, :] = f(p) * u + 0.5 * torch.randn(H, d, generator=g)
    kc = workloads.key_pool(kc)
    key = wl.key.float().cpu()
    qsl = np.concatenate([[0], np.cumsum(wl.num_scheduled_tokens)])
    for r, f in enumerate(growth):
        for t in range(int(wl.num_scheduled_tokens[r])):
            key[qsl[r] + t] = f(int(wl.num_computed_tokens[r]) + t) * u + \
                0.5 * torch.randn(H, d, generator=g)
    q = u.repeat_interleave(G, 0)[None] + 0.5 * torch.randn(wl.num_tokens, H * G, d, generator=g)
    dev = wl.key_cache.device
    wl.key_cache = kc.to(wl.dtype).to(dev)
    wl.key = key.to(wl.dtype).to(dev)
    wl.q = q.to(wl.dtype).to(dev)
    return wl


@pytest.mark.parametrize("split_tokens", [0, 64])
def test_attention_scores_that_keep_growing(split_tokens):
    """Scores that grow by about 20 log2 units every 32 keys (twice the lazy
    rescale bound per half step of a prompt tile), fall, or spike at sparse
    positions: prompt chunks and decodes against the fp64 oracle."""
    wl = workloads.build("grow", [150, 1, 100, 1, 70], [200, 700, 0, 900, 330], num_q_heads=16,
                         num_kv_heads=4, head_dim=128, seed=61, device=device(), pool_slack=1.2)
    growth = [lambda p: 0.04 * p, lambda p: 0.04 * p, lambda p: 3.0 if p % 37 == 5 else -0.2,
              lambda p: 30.0 - 0.03 * p, lambda p: 0.02 * p * (1 if (p // 40) % 2 else -1)]
    wl = _shape_scores(wl, growth, 62)
    _, _, _, out = gpu_step(wl, split_tokens=split_tokens)
    _, _, _, ref = oracle_step(wl)
    assert torch.isfinite(out).all()
    assert_attention_close(out, ref, wl.dtype, f"growing scores split {split_tokens}")
