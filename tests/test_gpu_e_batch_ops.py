"""GPU parity of the batch-side operations around the hot path, through the C
ABI, bit-exact against the oracle on the same seeded inputs:

- pkv_prepare_input_ids: the token-id gather of "Building the Batch" ("How
  they are computed") and the discard mask of "vLLM's Model Runner -- the
  Persistent Batch, in Source" ("The batch contains rows that must not be
  sampled");
- pkv_copy_blocks / pkv_zero_blocks: copy-on-write of a shared block ("How
  vLLM Works Internally: A Deep Dive", "Copy-on-Write for Beam Search") and
  clearing of fresh blocks ("Inside vLLM: Following One Request from the API to
  GPU Execution", Part 2, new_block_ids_to_zero).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import binding, workloads

from gpu_helpers import (assert_attention_close, bits_view, device, gpu_prepare, gpu_scales,
                         log)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prepare_page_examples.json")


def _i32(a, dev):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.int32))).to(dev)


def _batch(rng, R, max_new, row_width):
    """Seeded request state: scheduled and computed counts that fit the table
    row, a known total per request (some requests still mid-prompt, some done),
    and the token table."""
    nst = rng.integers(1, max_new + 1, R).astype(np.int32)
    nst[rng.random(R) < 0.5] = 1                     # decodes
    nct = np.array([rng.integers(0, row_width - n + 1) for n in nst], np.int32)
    total = np.minimum(nct + nst + rng.integers(-2, 40, R), row_width).astype(np.int32)
    table = rng.integers(0, 152064, (R, row_width)).astype(np.int32)
    return nst, nct, total, table


def _gpu_input_ids(nst, nct, total, table, *, with_token_indices=True, num_tokens=None):
    dev = device()
    R = len(nst)
    bt = torch.zeros((R, 1), dtype=torch.int32, device=dev)
    T = int(np.sum(nst)) if num_tokens is None else num_tokens
    prep = pkv.prepare_inputs(_i32(nst, dev), _i32(nct, dev), bt, num_tokens=T,
                              block_size=1 << 20, num_blocks=1)
    got = pkv.prepare_input_ids(_i32(table, dev), prep["req_indices"], prep["positions"],
                                prep["seq_lens"], _i32(total, dev),
                                with_token_indices=with_token_indices)
    torch.cuda.synchronize()
    return prep, got


def _oracle_input_ids(nst, nct, total, table):
    R = len(nst)
    ref = oracle.prepare(nst, nct, np.zeros((R, 1), np.int32), block_size=1 << 20, num_blocks=1)
    return oracle.input_ids(table, ref["req_indices"], ref["positions"], ref["seq_lens"], total)


def _assert_ids_equal(got, ref, what):
    assert np.array_equal(got["input_ids"].cpu().numpy(), ref["input_ids"]), f"{what}: input_ids"
    assert np.array_equal(got["discard_request_mask"].cpu().numpy(),
                          ref["discard_request_mask"]), f"{what}: discard mask"
    if "token_indices" in got:
        assert np.array_equal(got["token_indices"].cpu().numpy(), ref["token_indices"]), \
            f"{what}: token_indices"


def test_input_ids_page_examples():
    g = json.load(open(GOLDEN))
    e = g["token_indices_example"]
    M = 1000
    table = (np.arange(3 * M, dtype=np.int32) * 7 + 5).reshape(3, M)
    prep, got = _gpu_input_ids([2, 5, 3], [0, 0, 0], [2, 5, 3], table)
    assert prep["positions"].tolist() == e["positions"]
    want = [a * M + b for a, b in e["token_indices_in_units_of_M"]]
    assert got["token_indices"].tolist() == want
    e = g["discard_mask_example"]
    _, got = _gpu_input_ids(e["num_scheduled_tokens"], e["num_computed_tokens"],
                            e["num_tokens_total"], np.zeros((3, 700), np.int32))
    assert got["discard_request_mask"].bool().tolist() == e["discard_request_mask"]


@pytest.mark.parametrize("seed", range(6))
def test_input_ids_random_vs_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    R = int(rng.choice([1, 3, 255, 256, 257, 700]))
    row_width = int(rng.choice([64, 333, 4096]))
    nst, nct, total, table = _batch(rng, R, 40, row_width)
    log(f"input_ids seed={seed} R={R} T={int(nst.sum())} M={row_width}")
    _, got = _gpu_input_ids(nst, nct, total, table, with_token_indices=bool(seed % 2))
    _assert_ids_equal(got, _oracle_input_ids(nst, nct, total, table), f"seed {seed}")


def test_input_ids_large_step():
    """The token counts of a mixed step (one 5000-token chunk at position 3000
    plus 200 decodes at up to 8192) in a 201 x 8192 table: rows span many
    workgroups and end in a ragged tail."""
    rng = np.random.default_rng(77)
    nst = np.array([5000] + [1] * 200, np.int32)
    nct = np.array([3000] + list(rng.integers(1023, 8192, 200)), np.int32)
    total = nct + nst
    total[0] = 9000                                   # the chunk is mid-prompt
    table = rng.integers(0, 152064, (201, 8192)).astype(np.int32)
    _, got = _gpu_input_ids(nst, nct, total, table)
    ref = _oracle_input_ids(nst, nct, total, table)
    _assert_ids_equal(got, ref, "mixed step")
    assert ref["discard_request_mask"][0] == 1 and ref["discard_request_mask"][1:].sum() == 0


def test_input_ids_padding_rows_and_empty():
    """Rows past the device token total (pkv_prepare_inputs writes -1 there)
    get token index and id -1; an empty step launches nothing."""
    rng = np.random.default_rng(9)
    nst, nct, total, table = _batch(rng, 5, 6, 128)
    T = int(nst.sum())
    _, got = _gpu_input_ids(nst, nct, total, table, num_tokens=T + 37)
    ref = _oracle_input_ids(nst, nct, total, table)
    assert np.array_equal(got["input_ids"][:T].cpu().numpy(), ref["input_ids"])
    assert (got["input_ids"][T:] == -1).all() and (got["token_indices"][T:] == -1).all()
    _, got = _gpu_input_ids(np.zeros(0, np.int32), np.zeros(0, np.int32),
                            np.zeros(0, np.int32), np.zeros((0, 8), np.int32))
    assert got["input_ids"].numel() == 0 and got["discard_request_mask"].numel() == 0


# ---------------------------------------------------------------------------
# block copy / zeroing
# ---------------------------------------------------------------------------

POOLS = [  # (num_blocks, Hkv, d, dtype): block sizes below, at and above one 16 KiB chunk
    (40, 1, 64, torch.float32),      # 4 KiB per pool block
    (33, 3, 80, torch.bfloat16),     # 7.5 KiB: one partial chunk
    (50, 8, 128, torch.bfloat16),    # 32 KiB: two chunks
    (24, 8, 128, "fp8"),             # 16 KiB FP8 blocks
    (17, 40, 128, torch.bfloat16),   # 160 KiB: ten chunks
]


def _pools(nb, H, d, dtype, seed, bs=16):
    g = torch.Generator().manual_seed(seed)
    if dtype == "fp8":
        kc = torch.randint(0, 256, (nb, H, d * bs), generator=g, dtype=torch.uint8)
        vc = torch.randint(0, 256, (nb, H, d * bs), generator=g, dtype=torch.uint8)
    else:
        kc = torch.randn(nb, H, d * bs, generator=g).to(dtype)
        vc = torch.randn(nb, H, d * bs, generator=g).to(dtype)
    return kc, vc


def _cow_pairs(rng, nb, n):
    """n (source, destination) pairs: distinct destinations, none of them a
    source; sources drawn with repeats (one block forked to several beams)."""
    ids = rng.permutation(nb)
    dst = ids[:n]
    src = rng.choice(ids[n:], size=n, replace=True)
    return np.stack([src, dst], 1).astype(np.int32)


def _same_bits(a, b):
    return torch.equal(bits_view(a.cpu()), bits_view(b))


@pytest.mark.parametrize("case", range(len(POOLS)))
def test_copy_blocks_vs_oracle(case):
    nb, H, d, dtype = POOLS[case]
    rng = np.random.default_rng(600 + case)
    kc0, vc0 = _pools(nb, H, d, dtype, 600 + case)
    for n in (1, nb // 3, nb // 2):
        pairs = _cow_pairs(rng, nb, n)
        log(f"copy_blocks case={case} n={n}")
        kc, vc = kc0.to(device()), vc0.to(device())
        pkv.copy_blocks(kc, vc, _i32(pairs, device()))
        okc, ovc = kc0.clone(), vc0.clone()
        oracle.copy_blocks(okc, ovc, pairs)
        torch.cuda.synchronize()
        assert _same_bits(kc, okc) and _same_bits(vc, ovc), f"case {case} n {n}"


@pytest.mark.parametrize("case", range(len(POOLS)))
def test_zero_blocks_vs_oracle(case):
    nb, H, d, dtype = POOLS[case]
    rng = np.random.default_rng(700 + case)
    kc0, vc0 = _pools(nb, H, d, dtype, 700 + case)
    ids = rng.integers(0, nb, size=max(1, nb // 2)).astype(np.int32)   # with repeats
    kc, vc = kc0.to(device()), vc0.to(device())
    pkv.zero_blocks(kc, vc, _i32(ids, device()))
    okc, ovc = kc0.clone(), vc0.clone()
    oracle.zero_blocks(okc, ovc, ids)
    torch.cuda.synchronize()
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)


def test_block_ops_skip_ids_outside_the_pool_and_empty_lists():
    nb, H, d = 12, 2, 64
    kc0, vc0 = _pools(nb, H, d, torch.bfloat16, 3)
    kc, vc = kc0.to(device()), vc0.to(device())
    pkv.copy_blocks(kc, vc, _i32([[3, nb], [-1, 4], [2, 5]], device()))
    pkv.zero_blocks(kc, vc, _i32([nb, -7, 9], device()))
    pkv.copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device=device()))
    pkv.zero_blocks(kc, vc, torch.zeros(0, dtype=torch.int32, device=device()))
    okc, ovc = kc0.clone(), vc0.clone()
    oracle.copy_blocks(okc, ovc, [[2, 5]])
    oracle.zero_blocks(okc, ovc, [9])
    torch.cuda.synchronize()
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)


def test_copy_blocks_full_pool():
    """A bulk fork at the 32-head, 8-kv-head, d 128 bf16 pool geometry: 4096 of
    16384 blocks (32 KiB per pool block) copied to fresh blocks, checked
    against the oracle over the whole pools."""
    nb, H, d = 16384, 8, 128
    rng = np.random.default_rng(11)
    g = torch.Generator(device=device()).manual_seed(11)
    kc = torch.randint(-32768, 32767, (nb, H, 16, d), generator=g, device=device(),
                       dtype=torch.int16).view(torch.bfloat16)
    vc = torch.randint(-32768, 32767, (nb, H, d, 16), generator=g, device=device(),
                       dtype=torch.int16).view(torch.bfloat16)
    okc, ovc = kc.cpu(), vc.cpu()
    pairs = _cow_pairs(rng, nb, 4096)
    pkv.copy_blocks(kc, vc, _i32(pairs, device()))
    oracle.copy_blocks(okc, ovc, pairs)
    ids = rng.permutation(nb)[:2048].astype(np.int32)
    pkv.zero_blocks(kc, vc, _i32(ids, device()))
    oracle.zero_blocks(okc, ovc, ids)
    torch.cuda.synchronize()
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)


@pytest.mark.parametrize("fp8", [False, True])
def test_copy_on_write_beam_fork(fp8):
    """Four beams share a 40-token prefix (blocks 0..2, the last one partly
    filled).  Beams 1..3 copy the partial block to fresh blocks, point their
    tables there and each write a different next token at position 40; beam 0
    writes into the shared block itself.  Every beam's attention must equal
    the oracle's over the same pools, and beam 0's must not change when the
    copies are written."""
    dev = device()
    H, d, bs, L = 2, 128, 16, 40
    wl = workloads.build("cow", [1, 1, 1, 1], [L, L, L, L], num_q_heads=4, num_kv_heads=H,
                         head_dim=d, seed=31, device=dev, pool_slack=1.0, extra_table_cols=0)
    if fp8:
        wl = workloads.to_fp8(wl, 0.0125, 0.0125)
    ks, vs = gpu_scales(wl)
    nb = wl.key_cache.shape[0]
    shared = wl.block_table[0].copy()
    fresh = [b for b in range(nb) if b not in set(shared.tolist())][:3]
    assert len(fresh) == 3, "pool too small for the fork"
    bt = np.stack([shared] * 4)
    for beam in (1, 2, 3):
        bt[beam, 2] = fresh[beam - 1]
    wl.block_table = bt
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    pairs = np.array([[shared[2], f] for f in fresh], np.int32)
    pkv.copy_blocks(kc, vc, _i32(pairs, dev))
    prep, bt_dev = gpu_prepare(wl)
    if fp8:
        pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], ks, vs,
                               block_size=bs)
    else:
        pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=bs)
    out = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt_dev,
                              max_query_len=1, max_seq_len=L + 1, scale=wl.scale,
                              k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    okc, ovc = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
    oracle.copy_blocks(okc, ovc, pairs)
    slots = [int(bt[b, L // bs]) * bs + L % bs for b in range(4)]
    assert prep["slot_mapping"].tolist() == slots
    if fp8:
        oracle.kv_write_fp8(wl.key.cpu(), wl.value.cpu(), okc, ovc, slots, bs, *wl.kv_scales)
    else:
        oracle.kv_write(wl.key.cpu(), wl.value.cpu(), okc, ovc, slots, bs)
    assert _same_bits(kc, okc) and _same_bits(vc, ovc)
    ref = oracle.attention(wl.q.cpu(), okc, ovc, [0, 1, 2, 3, 4], [L + 1] * 4, bt, bs, wl.scale,
                           kv_scales=wl.kv_scales)
    assert_attention_close(out, ref, wl.dtype, "beam fork")
    # beam 0 alone, before the forks wrote their copies, sees the same context
    k0, v0 = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
    if fp8:
        oracle.kv_write_fp8(wl.key.cpu()[:1], wl.value.cpu()[:1], k0, v0, slots[:1], bs,
                            *wl.kv_scales)
    else:
        oracle.kv_write(wl.key.cpu()[:1], wl.value.cpu()[:1], k0, v0, slots[:1], bs)
    alone = oracle.attention(wl.q.cpu()[:1], k0, v0, [0, 1], [L + 1], bt[:1], bs, wl.scale,
                             kv_scales=wl.kv_scales)
    assert np.array_equal(alone[0], ref[0])
