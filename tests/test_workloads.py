"""The seeded input generator builds what the configurations say (no GPU)."""
import numpy as np
import torch

from paged_kv_cache_prepare_amd import workloads


def test_config1_structure_and_poison():
    wl = workloads.config(1)
    assert wl.num_scheduled_tokens.tolist() == [2, 5, 3]
    assert wl.num_computed_tokens.tolist() == [14, 0, 9]
    assert wl.num_blocks == 16 and wl.block_size == 16
    assert (wl.num_q_heads, wl.num_kv_heads, wl.head_dim) == (4, 2, 64)
    assert wl.dtype == torch.float32 and abs(wl.scale - 0.125) < 1e-15
    used = wl.block_table[wl.block_table >= 0]
    assert len(used) == 3 and len(set(used.tolist())) == 3
    # history slots are finite, everything else in the pool is NaN
    assert wl.key_cache.shape == (16, 2, 64 * 16)
    k = workloads.key_logical(wl.key_cache, 64, 16)
    hist = int(np.isfinite(k[:, 0, :, 0].numpy()).sum())
    assert hist == 14 + 0 + 9
    assert torch.isnan(wl.key_cache).sum() == (16 * 16 - 23) * 2 * 64
    assert torch.isnan(wl.value_cache).sum() == (16 * 16 - 23) * 2 * 64
    assert wl.q.shape == (10, 4, 64) and torch.isfinite(wl.q).all()


def test_same_seed_same_inputs():
    a, b = workloads.config(1), workloads.config(1)
    assert np.array_equal(a.block_table, b.block_table)
    assert torch.equal(a.q, b.q) and torch.equal(a.key, b.key)


def test_shared_prefix_groups_share_physical_blocks():
    wl = workloads.build("t", [1, 1, 1, 2], [63, 63, 40, 0], num_q_heads=4, num_kv_heads=2,
                         head_dim=8, seed=3, shared_prefix_groups=[([0, 1], 32)])
    bt = wl.block_table
    assert np.array_equal(bt[0, :2], bt[1, :2])
    assert bt[0, 2] != bt[1, 2] and bt[0, 3] != bt[1, 3]
    rest = np.concatenate([bt[0, :4], bt[1, 2:4], bt[2, :3], bt[3, :1]])
    assert len(set(rest.tolist())) == len(rest)
    assert wl.notes["shared_blocks"] == 2


def test_large_config_structures():
    s4 = workloads.config_structure(4)
    assert s4["num_scheduled_tokens"].sum() == 5200 and len(s4["num_scheduled_tokens"]) == 201
    ctx = s4["num_computed_tokens"][1:] + 1
    assert ctx.min() >= 1024 and ctx.max() <= 8192
    s5 = workloads.config_structure(5)
    assert s5["num_scheduled_tokens"].sum() == 2064
    assert (s5["num_computed_tokens"][:16] + 1 == 32768).all()


def test_select_keeps_rows_of_chosen_requests():
    wl = workloads.build("t", [3, 1, 2], [5, 9, 0], num_q_heads=4, num_kv_heads=2, head_dim=8,
                         seed=4)
    sub = workloads.select(wl, [2, 0])
    assert sub.num_scheduled_tokens.tolist() == [2, 3]
    assert np.array_equal(sub.block_table, wl.block_table[[2, 0]])
    assert torch.equal(sub.q, torch.cat([wl.q[4:6], wl.q[0:3]]))
    assert sub.key_cache is wl.key_cache


def test_config_structure_geometry_matches_the_configs():
    wl = workloads.config(1)
    s = workloads.config_structure(1)
    assert (s["num_q_heads"], s["num_kv_heads"], s["head_dim"], s["dtype"]) == \
        (wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.dtype)
    for idx in (2, 3, 4, 5):
        s = workloads.config_structure(idx)
        name = workloads.CONFIG_NAMES[idx]
        assert f"Hq {s['num_q_heads']} / Hkv {s['num_kv_heads']}, d {s['head_dim']}" in name
        assert s["dtype"] == torch.bfloat16 and "bf16" in name


def test_value_pool_order_and_inverse():
    """value_pool puts logical element (dim, tok) of a (block, head) run at
    ((dim // 16) * (bs // 4) + tok // 4) * 64 + (dim % 16) * 4 + tok % 4 (plain
    [dim][tok] when 16 does not divide d or 4 does not divide bs), and
    value_logical undoes it."""
    for d, bs in ((128, 16), (64, 16), (32, 8), (8, 4), (16, 6)):
        logical = torch.arange(3 * 2 * d * bs, dtype=torch.float32).reshape(3, 2, d, bs)
        pool = workloads.value_pool(logical)
        assert pool.shape == (3, 2, d * bs)
        tiled = d % 16 == 0 and bs % 4 == 0
        for dim in (0, 1, d // 2, d - 1):
            for tok in (0, 3, bs - 1):
                e = (((dim // 16) * (bs // 4) + tok // 4) * 64 + (dim % 16) * 4 + tok % 4
                     if tiled else dim * bs + tok)
                assert torch.equal(pool[:, :, e], logical[:, :, dim, tok]), (d, bs, dim, tok)
        assert torch.equal(workloads.value_logical(pool, d, bs), logical)


def test_key_pool_order_and_inverse():
    """key_pool puts element (tok, dim) of a (block, head) run at
    ((dim / 32) * bs + tok) * 32 + dim % 32 (plain [tok][dim] when 32 does not
    divide d); key_logical undoes it."""
    for d, bs in ((64, 16), (128, 4), (8, 5)):
        logical = torch.arange(3 * 2 * bs * d, dtype=torch.float32).reshape(3, 2, bs, d)
        pool = workloads.key_pool(logical)
        assert pool.shape == (3, 2, d * bs)
        kw = 32 if d % 32 == 0 else d
        for tok in range(bs):
            for dim in range(d):
                at = ((dim // kw) * bs + tok) * kw + dim % kw
                assert torch.equal(pool[:, :, at], logical[:, :, tok, dim])
        assert torch.equal(workloads.key_logical(pool, d, bs), logical)


def test_fp8_key_pool_order():
    logical = torch.arange(2 * 16 * 128, dtype=torch.int32).reshape(1, 2, 16, 128)
    pool = workloads.fp8_key_pool(logical)
    for tok in range(16):
        for dim in range(128):
            assert torch.equal(pool[:, :, (dim // 64) * 1024 + tok * 64 + dim % 64],
                               logical[:, :, tok, dim])
