"""pkv_paged_attention_plan / pkv_paged_attention_run: one work list per
batch, then one run per model layer.  Every run must equal, bit for bit, the
one-call pkv_paged_attention_varlen* on the same inputs (the same kernels over
the same list), for 16-bit and FP8 pools; a new plan in the same workspace
serves a new batch; the checked build rejects a run over a list made for
another batch."""
import numpy as np
import pytest
import torch

import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import binding, workloads

from gpu_helpers import (assert_attention_close, bits_view, device, gpu_prepare, gpu_scales,
                         log, oracle_step)

pytestmark = pytest.mark.gpu

NST, NCT = [1, 1, 70, 3, 1, 1], [900, 40, 100, 20, 2000, 333]


def _layers(n, fp8=False, nst=NST, nct=NCT):
    """n layers of one batch: the same token counts, each layer its own seeded
    q, K/V rows, pools and block placement."""
    out = []
    for k in range(n):
        wl = workloads.build(f"layer{k}", nst, nct, num_q_heads=16, num_kv_heads=4, head_dim=128,
                             seed=300 + k, device=device(), pool_slack=1.2)
        out.append(workloads.to_fp8(wl, 0.0125, 0.02) if fp8 else wl)
    return out


def _write(wl):
    prep, bt = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    ks, vs = gpu_scales(wl)
    if ks is None:
        pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=16)
    else:
        pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], ks, vs,
                               block_size=16)
    return prep, bt, kc, vc, ks, vs


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("split", [64, 0])
def test_one_plan_many_layers(fp8, split):
    layers = _layers(3, fp8)
    wl0 = layers[0]
    prep0, *_ = _write(wl0)
    ws = pkv.paged_attention_plan(prep0["query_start_loc"], prep0["seq_lens"],
                                  num_tokens=wl0.num_tokens, num_q_heads=16, num_kv_heads=4,
                                  head_dim=128, max_query_len=wl0.max_query_len,
                                  max_seq_len=wl0.max_seq_len, split_tokens=split)
    for k, wl in enumerate(layers):
        prep, bt, kc, vc, ks, vs = _write(wl)
        kw = dict(max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, scale=wl.scale,
                  split_tokens=split, k_scale=ks, v_scale=vs)
        # qsl / seq_lens of this layer hold the same values the plan was made from
        run = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                                  planned=True, workspace=ws, **kw)
        run = run.clone()
        fused = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                                    **kw)
        torch.cuda.synchronize()
        assert torch.equal(bits_view(run), bits_view(fused)), f"layer {k}"
        if k == 2:
            _, _, _, ref = oracle_step(wl)
            assert_attention_close(run, ref, wl.dtype, f"planned layer {k}")
        log(f"  layer {k}: run over the shared plan equals the one-call attention")


def test_replanning_the_workspace_for_a_new_batch():
    a = _layers(1)[0]
    b = _layers(1, nst=[1, 1, 1, 40], nct=[5000, 17, 260, 0])[0]
    prep_a, bt_a, kc_a, vc_a, _, _ = _write(a)
    prep_b, bt_b, kc_b, vc_b, _, _ = _write(b)
    # a workspace large enough for both batches
    size = max(pkv.attention_workspace_bytes(w.num_reqs, w.num_tokens, 16, 4, 128,
                                             w.max_query_len, w.max_seq_len, 64)
               for w in (a, b))
    ws = torch.empty(size, dtype=torch.uint8, device=device())
    for wl, prep, bt, kc, vc in ((a, prep_a, bt_a, kc_a, vc_a), (b, prep_b, bt_b, kc_b, vc_b),
                                 (a, prep_a, bt_a, kc_a, vc_a)):
        pkv.paged_attention_plan(prep["query_start_loc"], prep["seq_lens"],
                                 num_tokens=wl.num_tokens, num_q_heads=16, num_kv_heads=4,
                                 head_dim=128, max_query_len=wl.max_query_len,
                                 max_seq_len=wl.max_seq_len, split_tokens=64, workspace=ws)
        kw = dict(max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, scale=wl.scale,
                  split_tokens=64)
        run = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                                  planned=True, workspace=ws, **kw).clone()
        fused = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                                    **kw)
        torch.cuda.synchronize()
        assert torch.equal(bits_view(run), bits_view(fused))


@pytest.mark.parametrize("fp8", [False, True])
def test_runs_that_claim_prompt_tiles(fp8):
    """A batch with more prompt tiles than the chip has CUs plus decode items:
    the resident prompt workgroups claim tiles from a counter in the
    workspace, together with helper workgroups placed after the decode
    items, and the run that claims last zeroes the counter.  Four runs over
    one plan must equal each other bit for bit (which workgroup computes a
    tile does not change its result) and the oracle, and out is pre-filled
    with NaN, so a tile that no run computed would show."""
    nst = [2000, 1, 1, 1, 3, 1]
    nct = [1500, 700, 3000, 90, 40, 1200]
    wl = workloads.build("claims", nst, nct, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         seed=77, device=device(), pool_slack=1.2)
    if fp8:
        wl = workloads.to_fp8(wl, 0.0125, 0.02)
    G = wl.num_q_heads // wl.num_kv_heads
    tiles = -(-nst[0] * G // 128) * wl.num_kv_heads
    assert tiles > torch.cuda.get_device_properties(0).multi_processor_count
    prep, bt, kc, vc, ks, vs = _write(wl)
    ws = pkv.paged_attention_plan(prep["query_start_loc"], prep["seq_lens"],
                                  num_tokens=wl.num_tokens, num_q_heads=32, num_kv_heads=8,
                                  head_dim=128, max_query_len=wl.max_query_len,
                                  max_seq_len=wl.max_seq_len)
    kw = dict(max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, scale=wl.scale,
              k_scale=ks, v_scale=vs)
    outs = []
    for k in range(4):
        out = torch.full_like(wl.q, float("nan"))
        pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                            planned=True, workspace=ws, out=out, **kw)
        outs.append(out)
    torch.cuda.synchronize()
    for k in range(1, 4):
        assert torch.equal(bits_view(outs[k]), bits_view(outs[0])), f"run {k}"
    T = wl.num_tokens
    rows = np.array(sorted(set(range(0, T, 37)) | {T - 1} | set(range(nst[0], T))), np.int32)
    _, _, _, ref = oracle_step(wl, rows=rows)
    got = outs[0][torch.from_numpy(rows).long().to(device())]
    assert torch.isfinite(outs[0].float()).all()
    assert_attention_close(got, ref, wl.dtype, "claimed prompt tiles")
    log(f"  {tiles} prompt tiles, 4 runs over one plan: identical, and equal to the oracle")


def test_fp32_plan_is_a_no_op_and_run_works():
    wl = workloads.config(1, device=device())
    prep, bt, kc, vc, _, _ = _write(wl)
    ws = pkv.paged_attention_plan(prep["query_start_loc"], prep["seq_lens"],
                                  num_tokens=wl.num_tokens, num_q_heads=4, num_kv_heads=2,
                                  head_dim=64, max_query_len=wl.max_query_len,
                                  max_seq_len=wl.max_seq_len, dtype=torch.float32)
    kw = dict(max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, scale=wl.scale)
    run = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                              planned=True, workspace=ws, **kw).clone()
    fused = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(bits_view(run), bits_view(fused))


def test_checked_build_rejects_a_stale_plan():
    a = _layers(1)[0]
    b = _layers(1, nst=[1, 2, 1, 1, 1, 1], nct=NCT)[0]   # the same requests, other counts
    prep_a, bt_a, kc_a, vc_a, _, _ = _write(a)
    prep_b, *_ = _write(b)
    binding.use_checked(True)
    try:
        size = max(pkv.attention_workspace_bytes(w.num_reqs, w.num_tokens, 16, 4, 128,
                                                 w.max_query_len, w.max_seq_len, 64)
                   for w in (a, b))
        ws = torch.empty(size, dtype=torch.uint8, device=device())
        kw = dict(max_query_len=a.max_query_len, max_seq_len=a.max_seq_len, scale=a.scale,
                  split_tokens=64)
        pkv.paged_attention_plan(prep_b["query_start_loc"], prep_b["seq_lens"],
                                 num_tokens=b.num_tokens, num_q_heads=16, num_kv_heads=4,
                                 head_dim=128, max_query_len=b.max_query_len,
                                 max_seq_len=b.max_seq_len, split_tokens=64, workspace=ws)
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attention(a.q, kc_a, vc_a, prep_a["query_start_loc"], prep_a["seq_lens"],
                                bt_a, planned=True, workspace=ws, **kw)
        assert e.value.status == binding.ERR_DEVICE_DATA and "plan" in binding.check_flags()
        pkv.paged_attention_plan(prep_a["query_start_loc"], prep_a["seq_lens"],
                                 num_tokens=a.num_tokens, num_q_heads=16, num_kv_heads=4,
                                 head_dim=128, max_query_len=a.max_query_len,
                                 max_seq_len=a.max_seq_len, split_tokens=64, workspace=ws)
        pkv.paged_attention(a.q, kc_a, vc_a, prep_a["query_start_loc"], prep_a["seq_lens"], bt_a,
                            planned=True, workspace=ws, **kw)
        torch.cuda.synchronize()
    finally:
        binding.use_checked(False)


# pkv_prepare_inputs_and_plan: prepare + plan of one step in one launch.
FUSED = {
    # name: (nst, nct, Hq, Hkv, dtype, split, host token count (None: exact))
    "mixed": (NST, NCT, 16, 4, torch.bfloat16, 0, None),
    "mixed_split64": (NST, NCT, 16, 4, torch.bfloat16, 64, None),
    "decodes": ([1] * 40, [100 + 37 * i for i in range(40)], 32, 8, torch.bfloat16, 0, None),
    "padded": ([2, 5, 3], [14, 0, 9], 8, 2, torch.bfloat16, 0, 13),
    "f32": ([2, 5, 3], [14, 0, 9], 4, 2, torch.float32, 0, None),
    "many": (None, None, 8, 2, torch.bfloat16, 64, None),
}


def _list_of(ws):
    w = ws.cpu()
    head = w[:256].view(torch.int32).numpy().copy()
    n = int(head[0])
    items = w[256:256 + 16 * n].view(torch.int32).numpy().reshape(n, 4)
    return head, sorted(map(tuple, items.tolist()))


@pytest.mark.parametrize("case", list(FUSED))
def test_prepare_and_plan_in_one_launch(case):
    """The fused call writes the index tensors of pkv_prepare_inputs bit for
    bit, and a work list with the same header words (item counts, record of
    the sizes, batch checksum, zeroed claim counters) and the same items, as
    a multiset, as pkv_paged_attention_plan over those tensors.  Attention
    over the fused list matches the oracle."""
    nst, nct, Hq, Hkv, dtype, split, host_T = FUSED[case]
    if case == "many":  # more requests than one ranking pass of the plan holds
        rng = np.random.default_rng(77)
        nst = [1] * 1100
        nst[5] = 40
        nct = rng.integers(16, 300, 1100).tolist()
    wl = workloads.build(f"fused_{case}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=128 if dtype == torch.bfloat16 else 64, dtype=dtype,
                         seed=500 + len(case), device=device(), pool_slack=1.2)
    dev = wl.q.device
    T = wl.num_tokens if host_T is None else host_T
    args = (torch.from_numpy(wl.num_scheduled_tokens).to(dev),
            torch.from_numpy(wl.num_computed_tokens).to(dev),
            torch.from_numpy(wl.block_table).to(dev))
    sizes = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=wl.head_dim,
                 max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len, dtype=dtype,
                 split_tokens=split)
    need = pkv.attention_workspace_bytes(wl.num_reqs, T, Hq, Hkv, wl.head_dim, wl.max_query_len,
                                         wl.max_seq_len, split, dtype)
    ws_a = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev)
    ws_b = ws_a.clone()
    prep_a = pkv.prepare_inputs(*args, num_tokens=T, block_size=16, num_blocks=wl.num_blocks,
                                qsl_len=wl.num_reqs + 3)
    pkv.paged_attention_plan(prep_a["query_start_loc"][:wl.num_reqs + 1], prep_a["seq_lens"],
                             num_tokens=T, workspace=ws_a, **sizes)
    prep_b, ws = pkv.prepare_inputs_and_plan(*args, num_tokens=T, block_size=16,
                                             num_blocks=wl.num_blocks, workspace=ws_b,
                                             qsl_len=wl.num_reqs + 3, **sizes)
    torch.cuda.synchronize()
    assert ws is ws_b
    for k in prep_a:
        assert torch.equal(prep_a[k], prep_b[k]), f"{case}: {k} differs"
    if dtype != torch.bfloat16:
        assert bool((ws_b == 0xFF).all()), f"{case}: the fp32 path wrote the workspace"
        return
    head_a, items_a = _list_of(ws_a)
    head_b, items_b = _list_of(ws_b)
    words = [0, 1, 2, 4] + list(range(32, 41))
    assert head_a[words].tolist() == head_b[words].tolist(), f"{case}: list header differs"
    assert items_a == items_b, f"{case}: list items differ"
    assert head_b[0] > 0
    if case in ("many", "padded"):
        # the request-order list itself is checked by the plan coverage tests;
        # a run must use the plan's token count, which for "padded" is not q's
        return
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep_b["slot_mapping"], block_size=16)
    out = torch.full_like(wl.q, float("nan"))
    pkv.paged_attention(wl.q, kc, vc, prep_b["query_start_loc"][:wl.num_reqs + 1],
                        prep_b["seq_lens"], args[2], max_query_len=wl.max_query_len,
                        max_seq_len=wl.max_seq_len, scale=wl.scale, out=out,
                        split_tokens=split, workspace=ws_b, planned=True)
    torch.cuda.synchronize()
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, wl.dtype, f"fused {case}")
