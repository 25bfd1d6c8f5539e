"""A whole step (prepare -> kv write -> attention) captured in a HIP graph and
replayed: every replay must reproduce the eager result bit for bit, also after
the inputs are rewritten in place between replays ("How vLLM Works
Internally: A Deep Dive", "CUDA Graphs": a fixed-shape step is recorded once
and replayed).  The library allocates nothing and clears nothing with memset,
so the step is capturable as is."""
import pytest
import torch

import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import bits_view, device, log

pytestmark = pytest.mark.gpu


def _buffers(wl, dev):
    T, R = wl.num_tokens, wl.num_reqs
    i32 = dict(dtype=torch.int32, device=dev)
    prep = {"req_indices": torch.empty(T, **i32), "positions": torch.empty(T, **i32),
            "slot_mapping": torch.empty(T, dtype=torch.int64, device=dev),
            "query_start_loc": torch.empty(R + 1, **i32), "seq_lens": torch.empty(R, **i32),
            "logits_indices": torch.empty(R, **i32)}
    ws = torch.empty(max(256, pkv.attention_workspace_bytes(
        R, T, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.max_query_len, wl.max_seq_len, 64,
        wl.dtype)), dtype=torch.uint8, device=dev)
    return prep, ws


@pytest.mark.parametrize("fused", [False, True])
def test_step_replays_in_a_hip_graph(fused):
    """fused: the step as the benchmark runs it, prepare and the work list in
    one launch (pkv_prepare_inputs_and_plan), then the write and a run over
    the list."""
    dev = device()
    # decodes that are split into partitions, a prompt chunk, a short multi-row decode
    wl = workloads.build("graph", [1, 1, 70, 3, 1], [900, 40, 100, 20, 2000], num_q_heads=16,
                         num_kv_heads=4, head_dim=128, seed=23, device=dev, pool_slack=1.2)
    nst = torch.from_numpy(wl.num_scheduled_tokens).to(dev)
    nct = torch.from_numpy(wl.num_computed_tokens).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    q, key, value = wl.q.clone(), wl.key.clone(), wl.value.clone()
    kc0, vc0 = wl.key_cache.clone(), wl.value_cache.clone()
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.empty_like(q)
    prep, ws = _buffers(wl, dev)

    def step():
        if fused:
            pkv.prepare_inputs_and_plan(nst, nct, bt, num_tokens=wl.num_tokens,
                                        block_size=wl.block_size, num_blocks=wl.num_blocks,
                                        num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                                        head_dim=wl.head_dim, max_query_len=wl.max_query_len,
                                        max_seq_len=wl.max_seq_len, split_tokens=64,
                                        workspace=ws, out=prep)
        else:
            pkv.prepare_inputs(nst, nct, bt, num_tokens=wl.num_tokens, block_size=wl.block_size,
                               num_blocks=wl.num_blocks, out=prep)
        pkv.kv_cache_write(key, value, kc, vc, prep["slot_mapping"], block_size=wl.block_size)
        pkv.paged_attention(q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                            max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                            scale=wl.scale, out=out, split_tokens=64, workspace=ws,
                            planned=fused)

    def eager_reference():
        kc.copy_(kc0)
        vc.copy_(vc0)
        step()
        torch.cuda.synchronize()
        return ({k: v.clone() for k, v in prep.items()}, kc.clone(), vc.clone(), out.clone())

    ref = eager_reference()
    # capture (torch warms up on a side stream first)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kc.copy_(kc0)
        vc.copy_(vc0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    kc.copy_(kc0)
    vc.copy_(vc0)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    for rep in range(6):
        if rep == 3:  # new activations of the same shapes, written in place
            q.copy_(torch.randn(q.shape, generator=gen, device=dev).to(q.dtype))
            key.copy_(torch.randn(key.shape, generator=gen, device=dev).to(key.dtype))
            value.copy_(torch.randn(value.shape, generator=gen, device=dev).to(value.dtype))
            ref = eager_reference()
        kc.copy_(kc0)
        vc.copy_(vc0)
        out.fill_(float("nan"))
        for v in prep.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rp, rk, rv, ro = ref
        for k in rp:
            assert torch.equal(prep[k], rp[k]), f"replay {rep}: {k}"
        assert torch.equal(bits_view(kc), bits_view(rk)), f"replay {rep}: K pool"
        assert torch.equal(bits_view(vc), bits_view(rv)), f"replay {rep}: V pool"
        assert torch.equal(bits_view(out), bits_view(ro)), f"replay {rep}: attention output"
        log(f"  replay {rep}: bit-identical to the eager step")
        # eager work between replays on the same stream
        eager_reference()


def test_input_prep_and_block_ops_replay_in_a_hip_graph():
    """The batch-side calls are capturable too: prepare -> input-id gather ->
    a block copy-on-write and a clear of fresh blocks -> KV write ->
    attention, captured once and replayed, every replay bit-identical to the
    eager sequence (the clear is a kernel, not a memset node)."""
    dev = device()
    wl = workloads.build("graph2", [1, 1, 30, 1], [500, 47, 64, 1300], num_q_heads=8,
                         num_kv_heads=2, head_dim=128, seed=29, device=dev, pool_slack=1.5)
    nb = wl.num_blocks
    used = set(wl.block_table[wl.block_table >= 0].tolist())
    spare = [b for b in range(nb) if b not in used]
    assert len(spare) >= 4
    nst = torch.from_numpy(wl.num_scheduled_tokens).to(dev)
    nct = torch.from_numpy(wl.num_computed_tokens).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    M = int(wl.max_seq_len) + 8
    g = torch.Generator(device=dev).manual_seed(3)
    table = torch.randint(0, 50000, (wl.num_reqs, M), generator=g, device=dev, dtype=torch.int32)
    total = torch.tensor((wl.num_scheduled_tokens + wl.num_computed_tokens + [0, 5, 0, 1])
                         .astype("int32"), device=dev)
    # copy a used block to a spare one, clear two other spare blocks
    pairs = torch.tensor([[int(wl.block_table[0, 0]), spare[0]]], dtype=torch.int32, device=dev)
    clear = torch.tensor(spare[1:3], dtype=torch.int32, device=dev)
    kc0, vc0 = wl.key_cache.clone(), wl.value_cache.clone()
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.empty_like(wl.q)
    prep, ws = _buffers(wl, dev)
    ids = {"input_ids": torch.empty(wl.num_tokens, dtype=torch.int32, device=dev),
           "discard_request_mask": torch.empty(wl.num_reqs, dtype=torch.uint8, device=dev),
           "token_indices": torch.empty(wl.num_tokens, dtype=torch.int64, device=dev)}

    def step():
        pkv.prepare_inputs(nst, nct, bt, num_tokens=wl.num_tokens, block_size=wl.block_size,
                           num_blocks=nb, out=prep)
        pkv.prepare_input_ids(table, prep["req_indices"], prep["positions"], prep["seq_lens"],
                              total, out=ids)
        pkv.copy_blocks(kc, vc, pairs)
        pkv.zero_blocks(kc, vc, clear)
        pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"],
                           block_size=wl.block_size)
        pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                            max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                            scale=wl.scale, out=out, split_tokens=64, workspace=ws)

    def eager_reference():
        kc.copy_(kc0)
        vc.copy_(vc0)
        step()
        torch.cuda.synchronize()
        return ({k: v.clone() for k, v in {**prep, **ids}.items()}, kc.clone(), vc.clone(),
                out.clone())

    ref = eager_reference()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kc.copy_(kc0)
        vc.copy_(vc0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    kc.copy_(kc0)
    vc.copy_(vc0)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        kc.copy_(kc0)
        vc.copy_(vc0)
        out.fill_(float("nan"))
        for v in list(prep.values()) + list(ids.values()):
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rp, rk, rv, ro = ref
        for k in rp:
            cur = prep[k] if k in prep else ids[k]
            assert torch.equal(cur, rp[k]), f"replay {rep}: {k}"
        assert torch.equal(bits_view(kc), bits_view(rk)), f"replay {rep}: K pool"
        assert torch.equal(bits_view(vc), bits_view(rv)), f"replay {rep}: V pool"
        assert torch.equal(bits_view(out), bits_view(ro)), f"replay {rep}: attention output"
        assert not bits_view(kc[spare[1]]).any() and not bits_view(vc[spare[2]]).any()
        assert torch.equal(bits_view(kc[spare[0]]), bits_view(kc0[int(wl.block_table[0, 0])]))
        log(f"  replay {rep}: bit-identical to the eager sequence")
        eager_reference()


# Padded token counts ("Building the Batch", "Padding, after all that": a
# captured step has a fixed token count, so a batch of 37 tokens runs in a
# 40-row step whose extra rows belong to no request and write nothing; "How
# vLLM Works Internally: A Deep Dive", "CUDA Graphs").  One graph is captured
# at 40 rows with host-side upper bounds, and then replayed for batches of
# different sizes written in place into the same device buffers.  Each
# replay is compared with the oracle on the real rows.
T_PAD = 40
PAD_BATCHES = [  # (num_scheduled_tokens, num_computed_tokens); sums 37, 23, 39
    ([1, 1, 30, 3, 2], [900, 40, 100, 20, 1500]),
    ([1, 0, 20, 1, 1], [850, 40, 60, 20, 1400]),   # request 1 idle this step
    ([2, 1, 34, 1, 1], [898, 39, 96, 19, 1500]),
]


def test_padded_step_replays_match_the_oracle():
    import numpy as np
    import oracle
    from gpu_helpers import assert_attention_close

    dev = device()
    nst0, nct0 = PAD_BATCHES[0]
    Hq, Hkv, d = 16, 4, 128
    # one pool and table for every batch: each later batch reads positions
    # below its own computed count (history present) or written this step
    wl = workloads.build("padded", nst0, nct0, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                         seed=41, device=dev, pool_slack=1.2)
    for nst, nct in PAD_BATCHES:
        assert sum(nst) <= T_PAD
        assert all(c <= c0 and c + s <= c0 + s0
                   for s, c, s0, c0 in zip(nst, nct, nst0, nct0))
    R, nb = wl.num_reqs, wl.num_blocks
    max_q, max_L = T_PAD, int(max(a + b for a, b in zip(nst0, nct0)))
    nst_d = torch.zeros(R, dtype=torch.int32, device=dev)
    nct_d = torch.zeros(R, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    q = torch.zeros(T_PAD, Hq, d, dtype=wl.dtype, device=dev)
    key = torch.zeros(T_PAD, Hkv, d, dtype=wl.dtype, device=dev)
    value = torch.zeros(T_PAD, Hkv, d, dtype=wl.dtype, device=dev)
    kc0, vc0 = wl.key_cache.clone(), wl.value_cache.clone()
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.empty_like(q)
    i32 = dict(dtype=torch.int32, device=dev)
    prep = {"req_indices": torch.empty(T_PAD, **i32), "positions": torch.empty(T_PAD, **i32),
            "slot_mapping": torch.empty(T_PAD, dtype=torch.int64, device=dev),
            "query_start_loc": torch.empty(R + 1, **i32), "seq_lens": torch.empty(R, **i32),
            "logits_indices": torch.empty(R, **i32)}
    ws = torch.empty(max(256, pkv.attention_workspace_bytes(R, T_PAD, Hq, Hkv, d, max_q, max_L)),
                     dtype=torch.uint8, device=dev)

    def step():
        pkv.prepare_inputs(nst_d, nct_d, bt, num_tokens=T_PAD, block_size=16, num_blocks=nb,
                           out=prep)
        pkv.kv_cache_write(key, value, kc, vc, prep["slot_mapping"], block_size=16)
        pkv.paged_attention(q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                            max_query_len=max_q, max_seq_len=max_L, scale=wl.scale, out=out,
                            workspace=ws)

    gen = torch.Generator(device=dev).manual_seed(43)

    def load_batch(k):
        """Batch k's counts and fresh activations, in place; padding rows of
        key / value hold large values that must never reach a pool."""
        nst, nct = PAD_BATCHES[k]
        nst_d.copy_(torch.tensor(nst, dtype=torch.int32))
        nct_d.copy_(torch.tensor(nct, dtype=torch.int32))
        for t in (q, key, value):
            t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(t.dtype))
        T = sum(nst)
        key[T:] = 1000.0
        value[T:] = -1000.0
        return nst, nct, T

    def reset():
        kc.copy_(kc0)
        vc.copy_(vc0)
        out.fill_(float("nan"))
        for v in prep.values():
            v.fill_(-7)

    # warm-up on a side stream, then capture at 40 rows
    load_batch(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep, k in enumerate([0, 1, 2, 0, 2, 1]):
        nst, nct, T = load_batch(k)
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {name: v.cpu().numpy() for name, v in prep.items()}
        got_k, got_v, got_out = kc.cpu(), vc.cpu(), out.cpu()
        # eager step between replays, and replay == eager bit for bit
        reset()
        step()
        torch.cuda.synchronize()
        for name, v in prep.items():
            assert np.array_equal(v.cpu().numpy(), got[name]), f"replay {rep}: {name} vs eager"
        assert torch.equal(bits_view(kc.cpu()), bits_view(got_k)), f"replay {rep}: K vs eager"
        assert torch.equal(bits_view(out.cpu()), bits_view(got_out)), f"replay {rep}: out vs eager"
        # the oracle on the real rows
        ref_prep = oracle.prepare(np.array(nst, np.int32), np.array(nct, np.int32),
                                  wl.block_table, 16, nb)
        for name in ("query_start_loc", "seq_lens", "logits_indices"):
            assert np.array_equal(got[name], ref_prep[name]), f"replay {rep}: {name}"
        for name in ("req_indices", "positions", "slot_mapping"):
            assert np.array_equal(got[name][:T], ref_prep[name]), f"replay {rep}: {name}"
            assert (got[name][T:] == -1).all(), f"replay {rep}: padding rows of {name}"
        okc, ovc = kc0.cpu().clone(), vc0.cpu().clone()
        oracle.kv_write(key[:T].cpu(), value[:T].cpu(), okc, ovc, ref_prep["slot_mapping"], 16)
        assert torch.equal(bits_view(got_k), bits_view(okc)), f"replay {rep}: K pool"
        assert torch.equal(bits_view(got_v), bits_view(ovc)), f"replay {rep}: V pool"
        ref = oracle.attention(q[:T].cpu(), okc, ovc, ref_prep["query_start_loc"],
                               ref_prep["seq_lens"], wl.block_table, 16, wl.scale)
        assert_attention_close(got_out[:T], ref, wl.dtype, f"replay {rep} ({T} of {T_PAD} rows)")
        assert torch.isnan(got_out[T:].float()).all(), f"replay {rep}: a padding row was written"
        log(f"  replay {rep}: batch {k} ({T} tokens in {T_PAD} rows) matches the oracle")
