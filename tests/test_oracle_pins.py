"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * values the pages print (tests/golden/prepare_page_examples.json, each entry
    cited to its page and section);
  * torch's own fp64 scaled-dot-product attention over the whole unpaged
    sequence (a library routine the oracle does not call), which also fixes
    the causal alignment of a chunk that starts mid-sequence and the GQA head
    grouping;
  * closed forms (two-key softmax, all-ones V, zero Q, position-0 rows);
  * invariants (block-permutation and request-permutation invariance, padding
    of query_start_loc, uniqueness of slots).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _k_slab(d):
    return 32 if d % 32 == 0 else d


def k_elem(d, bs, dim, tok):
    """Element of (dim, tok) inside one (block, head) K run: slabs of 32 dims,
    [dim / 32][tok][dim % 32] (one slab spans every dim when 32 does not
    divide d)."""
    kw = _k_slab(d)
    return ((dim // kw) * bs + tok) * kw + dim % kw


def k_pool(logical):
    """A K pool [nb, Hkv, d * bs] from its logical form [nb, Hkv, bs, d]."""
    nb, H, bs, d = logical.shape
    out = torch.empty(nb, H, d * bs, dtype=logical.dtype)
    for dim in range(d):
        for tok in range(bs):
            out[:, :, k_elem(d, bs, dim, tok)] = logical[:, :, tok, dim]
    return out


def k_logical(pool, d, bs):
    """The logical [nb, Hkv, bs, d] view of a K pool (a copy)."""
    flat = pool.reshape(pool.shape[0], pool.shape[1], d * bs)
    out = torch.empty(pool.shape[0], pool.shape[1], bs, d, dtype=pool.dtype)
    for dim in range(d):
        for tok in range(bs):
            out[:, :, tok, dim] = flat[:, :, k_elem(d, bs, dim, tok)]
    return out


def _v_tiles(d, bs):
    return (16 if d % 16 == 0 else d), (4 if bs % 4 == 0 else bs)


def v_elem(d, bs, dim, tok):
    """Element of (dim, tok) inside one (block, head) V run: tiles of 16 dims x
    4 tokens, [dim / 16][tok / 4][dim % 16][tok % 4] (one tile spans every dim
    when 16 does not divide d, every token when 4 does not divide bs)."""
    dw, tg = _v_tiles(d, bs)
    return ((dim // dw) * (bs // tg) + tok // tg) * dw * tg + (dim % dw) * tg + tok % tg


def v_pool(logical):
    """A V pool [nb, Hkv, d * bs] from its logical form [nb, Hkv, d, bs]."""
    nb, H, d, bs = logical.shape
    out = torch.empty(nb, H, d * bs, dtype=logical.dtype)
    for dim in range(d):
        for tok in range(bs):
            out[:, :, v_elem(d, bs, dim, tok)] = logical[:, :, dim, tok]
    return out


def v_logical(pool, d, bs):
    """The logical [nb, Hkv, d, bs] view of a V pool (a copy)."""
    flat = pool.reshape(pool.shape[0], pool.shape[1], d * bs)
    out = torch.empty(pool.shape[0], pool.shape[1], d, bs, dtype=pool.dtype)
    for dim in range(d):
        for tok in range(bs):
            out[:, :, dim, tok] = flat[:, :, v_elem(d, bs, dim, tok)]
    return out

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prepare_page_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _table(rows, width=None):
    width = width or max(len(r) for r in rows)
    t = np.full((len(rows), width), -1, np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    return t


# ---------------------------------------------------------------------------
# prepare
# ---------------------------------------------------------------------------

def test_prepare_worked_example_253(golden):
    g = golden["worked_example_253"]
    nst = g["num_scheduled_tokens"]
    bt = _table([[0], [1], [2]])
    out = oracle.prepare(nst, [0, 0, 0], bt, block_size=16, num_blocks=3)
    assert out["req_indices"].tolist() == g["req_indices"]
    assert out["query_start_loc"][1:].tolist() == g["cu_num_tokens"]
    # with nothing computed yet a token's position is its offset in the chunk
    assert out["positions"].tolist() == g["query_pos"]
    assert out["query_start_loc"].tolist() == g["query_start_loc"]
    assert out["logits_indices"].tolist() == g["logits_indices"]


def test_prepare_positions_add_computed_tokens(golden):
    # "A token's position is its request's num_computed_tokens plus its offset
    # within this step's chunk" (Building the Batch, "How they are computed").
    g = golden["worked_example_253"]
    nct = [14, 0, 9]
    bt = _table([[5], [3], [9]])
    out = oracle.prepare(g["num_scheduled_tokens"], nct, bt, block_size=16, num_blocks=16)
    qpos = np.array(g["query_pos"])
    req = np.array(g["req_indices"])
    assert out["positions"].tolist() == (np.array(nct)[req] + qpos).tolist()
    assert out["seq_lens"].tolist() == [16, 5, 12]


def test_prepare_packed_batch_411(golden):
    g = golden["packed_batch_411"]
    bt = _table([[0], [1, 2, 3, 4], [5, 6]])
    out = oracle.prepare(g["num_scheduled_tokens"], g["num_computed_tokens"], bt,
                         block_size=16, num_blocks=8)
    assert out["positions"].tolist() == g["positions"]
    assert out["query_start_loc"].tolist() == g["query_start_loc"]


def test_prepare_go_program_hand_checked_slots(golden):
    g = golden["go_program_bs4"]
    bt = _table(g["block_tables"])
    out = oracle.prepare(g["num_scheduled_tokens"], g["num_computed_tokens"], bt,
                         block_size=g["block_size"], num_blocks=16)
    rows_b = np.nonzero(out["req_indices"] == 1)[0]
    assert out["positions"][rows_b].tolist() == g["request_B_positions"]
    assert out["slot_mapping"][rows_b].tolist() == g["request_B_slots"]


def test_prepare_nano_block_mapping(golden):
    g = golden["nano_block_mapping"]
    bs = g["block_size"]
    out = oracle.prepare([10], [0], _table([g["block_table"]]), block_size=bs, num_blocks=16)
    slots = out["slot_mapping"]
    assert (slots // bs).tolist() == g["token_physical_block"]
    assert (slots % bs).tolist() == g["token_in_block_order"]


def test_prepare_hand_derived_exercises(golden):
    h = golden["hand_derived"]
    q2 = h["check_yourself_q2"]
    # a single decode token at position 37
    out = oracle.prepare([1], [q2["position"]], _table([q2["block_table"]]),
                         block_size=q2["block_size"], num_blocks=64)
    assert out["slot_mapping"].tolist() == [q2["slot"]]
    t1 = h["try_it_q1"]
    out = oracle.prepare([t1["num_scheduled_tokens"]], [t1["num_computed_tokens"]],
                         _table([t1["block_table"]]), block_size=t1["block_size"], num_blocks=16)
    assert out["slot_mapping"].tolist() == t1["slots"]


def test_prepare_new_block_exactly_at_boundary():
    # nano-vLLM section 2.6: a decode step needs a fresh block exactly when
    # len(seq) % block_size == 1, i.e. the new token is the first of a block.
    bs = 16
    lens = np.arange(1, 100)
    nct = lens - 1
    R = len(lens)
    need = (lens + bs - 1) // bs
    bt = np.full((R, need.max()), -1, np.int32)
    for r in range(R):
        bt[r, :need[r]] = 1000 + 10 * r + np.arange(need[r])
    out = oracle.prepare(np.ones(R), nct, bt, block_size=bs, num_blocks=10_000)
    first_of_block = (out["slot_mapping"] % bs) == 0
    assert first_of_block.tolist() == ((lens % bs) == 1).tolist()
    # and the block it lands in is the request's last table entry
    assert (out["slot_mapping"] // bs).tolist() == [bt[r, need[r] - 1] for r in range(R)]


def test_prepare_query_start_loc_tail_padding():
    # "the unused tail is filled with the total so that every request beyond
    # the real ones has zero length" (Building the Batch, "How they are computed")
    out = oracle.prepare([3, 1, 4], [0, 7, 2], _table([[0], [1], [2]]), block_size=16,
                         num_blocks=3, qsl_len=9)
    qsl = out["query_start_loc"]
    assert qsl.tolist() == [0, 3, 4, 8, 8, 8, 8, 8, 8]
    assert np.all(np.diff(qsl) >= 0)


@pytest.mark.parametrize("seed", range(6))
def test_prepare_random_matches_vectorised_form_and_invariants(seed):
    """Loop oracle vs the pages' vectorised NumPy form (np.repeat / cumsum /
    fancy indexing, as printed in "How they are computed"), plus invariants."""
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 12))
    bs = int(rng.choice([1, 4, 16]))
    nst = rng.integers(0, 40, size=R).astype(np.int32)
    nct = rng.integers(0, 70, size=R).astype(np.int32)
    seq = nst + nct
    need = (seq + bs - 1) // bs
    nb = int(need.sum()) + 5
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((R, max(int(need.max()), 1) + 2), -1, np.int32)
    c = 0
    for r in range(R):
        bt[r, :need[r]] = perm[c:c + need[r]]
        c += need[r]
    out = oracle.prepare(nst, nct, bt, block_size=bs, num_blocks=nb, qsl_len=R + 3)
    T = int(nst.sum())

    req = np.repeat(np.arange(R), nst)
    cu = np.cumsum(nst)
    query_pos = np.arange(T) - np.repeat(cu - nst, nst)
    pos = nct[req] + query_pos
    slots = bt[req, pos // bs].astype(np.int64) * bs + pos % bs
    assert out["req_indices"].tolist() == req.tolist()
    assert out["positions"].tolist() == pos.tolist()
    assert out["slot_mapping"].tolist() == slots.tolist()
    assert out["query_start_loc"].tolist() == [0] + cu.tolist() + [T, T]
    assert out["seq_lens"].tolist() == seq.tolist()
    # invariants
    qsl = out["query_start_loc"]
    assert qsl[R] == T
    assert np.all(out["positions"] < out["seq_lens"][out["req_indices"]])
    q_len = qsl[1:R + 1] - qsl[:R]
    r_of = out["req_indices"]
    t = np.arange(T) - qsl[r_of]
    assert np.all(out["positions"] == out["seq_lens"][r_of] - q_len[r_of] + t)
    assert len(set(out["slot_mapping"].tolist())) == T  # disjoint tables -> unique slots


def test_prepare_rejects_out_of_range_blocks():
    with pytest.raises(oracle.OracleError) as e:
        oracle.prepare([2], [15], _table([[0]]), block_size=16, num_blocks=4)
    assert e.value.code == oracle.ERR_RANGE  # position 16 needs a second table column
    with pytest.raises(oracle.OracleError) as e:
        oracle.prepare([1], [0], _table([[9]]), block_size=16, num_blocks=4)
    assert e.value.code == oracle.ERR_RANGE


def test_prepare_empty_batch():
    out = oracle.prepare(np.zeros(0, np.int32), np.zeros(0, np.int32),
                         np.zeros((0, 1), np.int32), block_size=16, num_blocks=1, qsl_len=4)
    assert out["query_start_loc"].tolist() == [0, 0, 0, 0]
    assert out["slot_mapping"].size == 0


# ---------------------------------------------------------------------------
# kv_write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("nb,H,bs,d,T", [(7, 3, 4, 8, 9), (5, 2, 8, 32, 11)])
def test_kv_write_post_state(dtype, nb, H, bs, d, T):
    g = torch.Generator().manual_seed(3)
    kc = k_pool(torch.randn(nb, H, bs, d, generator=g).to(dtype))
    vc = v_pool(torch.randn(nb, H, d, bs, generator=g).to(dtype))
    key = torch.randn(T, H, d, generator=g).to(dtype)
    val = torch.randn(T, H, d, generator=g).to(dtype)
    slots = torch.randperm(nb * bs, generator=g)[:T].numpy().astype(np.int64)
    slots[4] = -1  # padding row: no write
    kc0, vc0 = kc.clone(), vc.clone()
    oracle.kv_write(key, val, kc, vc, slots, block_size=bs)
    kc, kc0 = k_logical(kc, d, bs), k_logical(kc0, d, bs)
    vc, vc0 = v_logical(vc, d, bs), v_logical(vc0, d, bs)
    written = np.zeros((nb, bs), bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), bs)
        written[b, o] = True
        assert torch.equal(kc[b, :, o, :], key[i])
        assert torch.equal(vc[b, :, :, o], val[i])
    keep = torch.from_numpy(~written)
    assert torch.equal(kc[keep[:, None, :, None].expand_as(kc)],
                       kc0[keep[:, None, :, None].expand_as(kc0)])
    assert torch.equal(vc[keep[:, None, None, :].expand_as(vc)],
                       vc0[keep[:, None, None, :].expand_as(vc0)])


def test_key_layout_positions():
    """Where one token's K row lands in the pool, element by element, for a
    slab run (head_dim 64, block_size 8) and a plain one (head_dim 8,
    block_size 6): the documented order written out, not k_elem."""
    for d, bs, slot, expect in (
            (64, 8, 2 * 8 + 5, lambda dim: (dim // 32) * 256 + 5 * 32 + dim % 32),
            (8, 6, 1 * 6 + 4, lambda dim: 4 * 8 + dim)):
        H = 2
        kc = torch.zeros(4, H, d * bs)
        vc = torch.zeros(4, H, d * bs)
        val = (torch.arange(H * d, dtype=torch.float32) + 1).reshape(1, H, d)
        oracle.kv_write(val, val, kc, vc, [slot], block_size=bs)
        blk = slot // bs
        for h in range(H):
            for dim in range(d):
                assert kc[blk, h, expect(dim)] == h * d + dim + 1, (d, bs, h, dim)
        assert int((kc != 0).sum()) == H * d


def test_key_layout_slabs_are_whole_lines():
    """In a 16-bit K run of head_dim 128 and a 16-token block, the 16 tokens x
    32 dims of one slab fill 8 aligned 128-byte lines and nothing else (one
    wave-wide 16-byte load), and one token's row lands in 4 runs of 64
    contiguous bytes."""
    d, bs = 128, 16
    for s in range(d // 32):
        byte_set = {k_elem(d, bs, dim, tok) * 2 // 128 for tok in range(bs)
                    for dim in range(32 * s, 32 * s + 32)}
        assert byte_set == set(range(8 * s, 8 * s + 8))
    for tok in range(bs):
        starts = sorted(k_elem(d, bs, dim, tok) for dim in range(0, d, 32))
        for dim0 in range(0, d, 32):
            run = [k_elem(d, bs, dim, tok) for dim in range(dim0, dim0 + 32)]
            assert run == list(range(run[0], run[0] + 32))
        assert len(starts) == 4


def test_value_layout_positions():
    """Where one token's V row lands in the pool, element by element, for a
    tiled run (head_dim 32, block_size 8) and an untiled one (head_dim 8,
    block_size 6): the documented order written out, not v_elem."""
    for d, bs, slot, expect in (
            (32, 8, 2 * 8 + 5, lambda dim: ((dim // 16) * 2 + 1) * 64 + (dim % 16) * 4 + 1),
            (8, 6, 1 * 6 + 4, lambda dim: dim * 6 + 4)):
        H = 2
        kc = torch.zeros(4, H, bs, d)
        vc = torch.zeros(4, H, d * bs)
        val = (torch.arange(H * d, dtype=torch.float32) + 1).reshape(1, H, d)
        oracle.kv_write(val, val, kc, vc, [slot], block_size=bs)
        blk = slot // bs
        for h in range(H):
            for dim in range(d):
                assert vc[blk, h, expect(dim)] == h * d + dim + 1, (d, bs, h, dim)
        assert int((vc != 0).sum()) == H * d


def test_value_layout_decode_row_lines():
    """A 16-bit decode row of head_dim 128 in a 16-token block lands in 8
    aligned 128-byte lines per head (16 dims x 4 tokens x 2 bytes each), the
    reason for the tiled V order: a partly written line costs a later
    write-back."""
    d, bs = 128, 16
    for tok in range(bs):
        lines = {v_elem(d, bs, dim, tok) * 2 // 128 for dim in range(d)}
        assert len(lines) == 8


def test_kv_write_rejects_duplicates_and_range():
    kc = torch.zeros(2, 1, 4, 8)
    vc = torch.zeros(2, 1, 8, 4)
    k = torch.ones(2, 1, 8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_write(k, k, kc, vc, [3, 3], block_size=4)
    assert e.value.code == oracle.ERR_DUP
    with pytest.raises(oracle.OracleError) as e:
        oracle.kv_write(k, k, kc, vc, [3, 8], block_size=4)
    assert e.value.code == oracle.ERR_RANGE


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def make_paged(nst, nct, Hq, Hkv, d, bs, seed, dtype=torch.float32, slack=3):
    """Contiguous per-request K/V/Q first, then the same rows placed into a
    NaN-filled paged pool at random blocks.  Returns (logical, paged)."""
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    nst = np.asarray(nst, np.int32)
    nct = np.asarray(nct, np.int32)
    R = len(nst)
    L = nst + nct
    need = (L + bs - 1) // bs
    nb = int(need.sum()) + slack
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((R, int(need.max()) + 1), -1, np.int32)
    c = 0
    for r in range(R):
        bt[r, :need[r]] = perm[c:c + need[r]]
        c += need[r]
    Ks = [torch.randn(int(L[r]), Hkv, d, generator=g).to(dtype) for r in range(R)]
    Vs = [torch.randn(int(L[r]), Hkv, d, generator=g).to(dtype) for r in range(R)]
    Qs = [torch.randn(int(L[r]), Hq, d, generator=g).to(dtype) for r in range(R)]
    kc = torch.full((nb, Hkv, bs, d), float("nan"), dtype=dtype)
    vc = torch.full((nb, Hkv, d, bs), float("nan"), dtype=dtype)
    for r in range(R):
        for j in range(int(L[r])):
            b, o = int(bt[r, j // bs]), j % bs
            kc[b, :, o, :] = Ks[r][j]
            vc[b, :, :, o] = Vs[r][j]
    kc = k_pool(kc)
    vc = v_pool(vc)
    q = torch.cat([Qs[r][int(nct[r]):] for r in range(R)]).contiguous()
    qsl = np.concatenate([[0], np.cumsum(nst)]).astype(np.int32)
    return dict(Ks=Ks, Vs=Vs, Qs=Qs, nst=nst, nct=nct), dict(
        q=q, kc=kc, vc=vc, qsl=qsl, seq_lens=L.astype(np.int32), bt=bt, bs=bs)


def sdpa_reference(logical, scale):
    """torch fp64 SDPA over each whole sequence (is_causal on the square
    L x L problem), keeping the rows of this step's chunk."""
    outs = []
    for Qr, Kr, Vr, n, c in zip(logical["Qs"], logical["Ks"], logical["Vs"],
                                logical["nst"], logical["nct"]):
        if n == 0:
            continue
        o = F.scaled_dot_product_attention(
            Qr.double().transpose(0, 1)[None], Kr.double().transpose(0, 1)[None],
            Vr.double().transpose(0, 1)[None], is_causal=True, scale=scale, enable_gqa=True)
        outs.append(o[0].transpose(0, 1)[int(c):])
    return torch.cat(outs).numpy()


def run_oracle(paged, scale, rows=None):
    return oracle.attention(paged["q"], paged["kc"], paged["vc"], paged["qsl"],
                            paged["seq_lens"], paged["bt"], paged["bs"], scale, rows=rows)


CASES = [
    # (nst, nct, Hq, Hkv, d, bs)
    ([1, 1, 1], [0, 5, 40], 4, 4, 16, 4),               # decodes incl. a position-0 token
    ([7, 1, 3], [0, 19, 9], 4, 2, 8, 4),                # fresh prefill, decode, chunk mid-seq
    ([2, 5, 3], [14, 0, 9], 4, 2, 64, 16),              # the worked-example shape
    ([33, 1, 0, 2], [17, 64, 5, 0], 8, 2, 32, 16),      # GQA 4, empty request, ragged
    ([5], [60], 6, 1, 16, 8),                           # MQA
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_matches_torch_sdpa(case):
    nst, nct, Hq, Hkv, d, bs = CASES[case]
    logical, paged = make_paged(nst, nct, Hq, Hkv, d, bs, seed=10 + case)
    scale = 1.0 / math.sqrt(d)
    ref = sdpa_reference(logical, scale)
    got = run_oracle(paged, scale)
    assert got.shape == ref.shape
    assert np.isfinite(got).all()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_scale_is_applied():
    logical, paged = make_paged([3, 1], [4, 9], 2, 2, 16, 4, seed=5)
    for scale in (0.05, 0.7):
        assert np.max(np.abs(run_oracle(paged, scale) - sdpa_reference(logical, scale))) < 1e-12


def test_attention_bf16_inputs_widen_exactly():
    logical, paged = make_paged([3, 1], [5, 30], 4, 2, 32, 16, seed=6, dtype=torch.bfloat16)
    scale = 0.125
    ref = sdpa_reference(logical, scale)   # bf16 values upcast exactly to fp64
    assert np.max(np.abs(run_oracle(paged, scale) - ref)) < 1e-12


def test_attention_two_key_closed_form():
    # one request, 2 tokens of history + 1 new token at position 2; head_dim 1
    # keys 0, 1, 2 with k = [1, 2, -1], q = 0.5, v = [10, 20, 30], scale 1
    # -> weights exp(0.5), exp(1.0), exp(-0.5) (closed form written out)
    kc = torch.full((1, 1, 4, 1), float("nan"))
    vc = torch.full((1, 1, 1, 4), float("nan"))
    kc[0, 0, :3, 0] = torch.tensor([1.0, 2.0, -1.0])
    vc[0, 0, 0, :3] = torch.tensor([10.0, 20.0, 30.0])
    q = torch.tensor([[[0.5]]])
    out = oracle.attention(q, kc, vc, [0, 1], [3], np.array([[0]]), 4, 1.0)
    w = np.exp([0.5, 1.0, -0.5])
    expect = (w @ np.array([10.0, 20.0, 30.0])) / w.sum()
    assert abs(out[0, 0, 0] - expect) < 1e-12


def test_attention_block_permutation_invariance():
    logical, paged = make_paged([6, 1, 2], [10, 33, 0], 4, 2, 16, 4, seed=7, slack=6)
    base = run_oracle(paged, 0.25)
    rng = np.random.default_rng(1)
    nb = paged["kc"].shape[0]
    perm = rng.permutation(nb)          # new position of old block b is perm[b]
    kc2 = torch.empty_like(paged["kc"])
    vc2 = torch.empty_like(paged["vc"])
    kc2[torch.from_numpy(perm)] = paged["kc"]
    vc2[torch.from_numpy(perm)] = paged["vc"]
    bt2 = np.where(paged["bt"] >= 0, perm[np.maximum(paged["bt"], 0)], -1).astype(np.int32)
    moved = dict(paged, kc=kc2, vc=vc2, bt=bt2)
    assert np.array_equal(run_oracle(moved, 0.25), base)   # bit-exact


def test_attention_request_permutation_permutes_rows():
    nst, nct = [3, 1, 2], [2, 20, 7]
    logical, paged = make_paged(nst, nct, 4, 2, 16, 4, seed=8)
    base = run_oracle(paged, 0.3)
    order = [2, 0, 1]
    qsl = paged["qsl"]
    row_blocks = [np.arange(qsl[r], qsl[r + 1]) for r in range(3)]
    new_rows = np.concatenate([row_blocks[r] for r in order])
    new_nst = np.array(nst)[order]
    moved = dict(paged, q=paged["q"][torch.from_numpy(new_rows)].contiguous(),
                 qsl=np.concatenate([[0], np.cumsum(new_nst)]).astype(np.int32),
                 seq_lens=paged["seq_lens"][order], bt=paged["bt"][order])
    assert np.array_equal(run_oracle(moved, 0.3), base[new_rows])


def test_attention_softmax_rows_sum_to_one():
    logical, paged = make_paged([4, 1], [3, 50], 4, 2, 16, 4, seed=9)
    ones_v = torch.where(torch.isnan(paged["vc"]), paged["vc"], torch.ones_like(paged["vc"]))
    out = oracle.attention(paged["q"], paged["kc"], ones_v, paged["qsl"], paged["seq_lens"],
                           paged["bt"], paged["bs"], 0.5)
    assert np.max(np.abs(out - 1.0)) < 1e-14


def test_attention_position_zero_returns_first_value():
    logical, paged = make_paged([5], [0], 2, 1, 16, 4, seed=11)
    out = run_oracle(paged, 0.25)
    v0 = logical["Vs"][0][0, 0].double().numpy()
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)


def test_attention_zero_query_averages_visible_values():
    logical, paged = make_paged([3, 1], [4, 12], 2, 2, 8, 4, seed=12)
    zq = dict(paged, q=torch.zeros_like(paged["q"]))
    out = run_oracle(zq, 0.7)
    row = 0
    for r in range(2):
        for t in range(int(logical["nst"][r])):
            p = int(logical["nct"][r]) + t
            mean = logical["Vs"][r][:p + 1].double().mean(0).numpy()   # [Hkv, d]
            assert np.max(np.abs(out[row] - mean)) < 1e-14
            row += 1


def test_attention_gqa_equals_mha_on_repeated_kv():
    nst, nct = [2, 1], [5, 9]
    logical, paged = make_paged(nst, nct, 6, 2, 8, 4, seed=13)
    gqa = run_oracle(paged, 0.4)
    rep = dict(paged, kc=paged["kc"].repeat_interleave(3, dim=1).contiguous(),
               vc=paged["vc"].repeat_interleave(3, dim=1).contiguous())
    mha = run_oracle(rep, 0.4)
    assert np.array_equal(gqa, mha)


def test_attention_row_subset_matches_full():
    logical, paged = make_paged([6, 1, 4], [3, 40, 0], 4, 2, 16, 4, seed=14)
    full = run_oracle(paged, 0.25)
    rows = np.array([10, 0, 7, 3])
    assert np.array_equal(run_oracle(paged, 0.25, rows=rows), full[rows])


def test_attention_rejects_bad_inputs():
    logical, paged = make_paged([2], [3], 2, 1, 8, 4, seed=15)
    with pytest.raises(oracle.OracleError) as e:   # q_len > seq_len
        oracle.attention(paged["q"], paged["kc"], paged["vc"], [0, 2], [1], paged["bt"], 4, 1.0)
    assert e.value.code == oracle.ERR_PRECOND
    bad = paged["bt"].copy()
    bad[0, 0] = 999
    with pytest.raises(oracle.OracleError) as e:
        oracle.attention(paged["q"], paged["kc"], paged["vc"], paged["qsl"], paged["seq_lens"],
                         bad, 4, 1.0)
    assert e.value.code == oracle.ERR_RANGE


def test_prepare_write_attention_chain_equals_unpaged_sdpa():
    """The three oracle steps chained the way one step of the hot path runs:
    prepare -> write the new rows at slot_mapping -> attention."""
    nst, nct = np.array([3, 1, 5], np.int32), np.array([6, 21, 0], np.int32)
    logical, paged = make_paged(nst, nct, 4, 2, 16, 4, seed=16)
    R = len(nst)
    # wipe this step's slots, then let prepare + kv_write put them back
    kc, vc = k_logical(paged["kc"], 16, 4), v_logical(paged["vc"], 16, 4)
    key = torch.cat([logical["Ks"][r][nct[r]:] for r in range(R)]).contiguous()
    val = torch.cat([logical["Vs"][r][nct[r]:] for r in range(R)]).contiguous()
    prep = oracle.prepare(nst, nct, paged["bt"], block_size=4, num_blocks=kc.shape[0])
    for s in prep["slot_mapping"]:
        kc[s // 4, :, s % 4, :] = float("nan")
        vc[s // 4, :, :, s % 4] = float("nan")
    kc, vc = k_pool(kc), v_pool(vc)
    oracle.kv_write(key, val, kc, vc, prep["slot_mapping"], block_size=4)
    out = oracle.attention(paged["q"], kc, vc, prep["query_start_loc"], prep["seq_lens"],
                           paged["bt"], 4, 0.25)
    assert np.max(np.abs(out - sdpa_reference(logical, 0.25))) < 1e-12


# ---------------------------------------------------------------------------
# FP8 cache ("How vLLM Works Internally: A Deep Dive", "FP8 KV Cache"; the
# write call's kv_cache_dtype / k_scale / v_scale, "Inside vLLM...", Part 5).
# The format is OCP FP8 E4M3; torch's float8_e4m3fn is an independent
# implementation of the same format.
# ---------------------------------------------------------------------------

def _fp8_table():
    return np.array([oracle.fp8_decode(c) for c in range(256)])


def test_fp8_decode_matches_torch_float8_e4m3fn_for_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = _fp8_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_format_landmarks():
    # largest finite 448 = 1.75 * 2^8, one = bias 7, smallest subnormal 2^-9,
    # no infinities: the all-ones codes are the only NaNs
    assert oracle.fp8_decode(0x7E) == 448.0 and oracle.fp8_decode(0xFE) == -448.0
    assert oracle.fp8_decode(0x38) == 1.0
    assert oracle.fp8_decode(0x01) == 2.0 ** -9 and oracle.fp8_decode(0x08) == 2.0 ** -6
    assert [c for c in range(256) if math.isnan(oracle.fp8_decode(c))] == [0x7F, 0xFF]


def test_fp8_encode_round_trips_every_code():
    for c in range(256):
        v = oracle.fp8_decode(c)
        if not math.isnan(v):
            assert oracle.fp8_encode(v) == c, hex(c)


def test_fp8_encode_is_nearest_with_ties_to_even():
    table = _fp8_table()
    finite = [c for c in range(256) if not math.isnan(table[c])]
    vals = np.array([table[c] for c in finite])
    rng = np.random.default_rng(3)
    # random magnitudes over the whole range, plus every exact midpoint
    xs = list(rng.standard_normal(4000) * 40) + list(rng.uniform(-2 ** -5, 2 ** -5, 2000))
    pos = np.unique(np.abs(vals))
    xs += list((pos[1:] + pos[:-1]) / 2) + list(-(pos[1:] + pos[:-1]) / 2)
    for x in xs:
        x32 = float(np.float32(x))
        c = oracle.fp8_encode(x32)
        v = oracle.fp8_decode(c)
        d = np.abs(vals - x32)
        best = d.min()
        assert abs(v - x32) == best, (x32, hex(c))
        ties = [finite[i] for i in np.nonzero(d == best)[0] if (finite[i] & 0x7F) or x32 == 0]
        if len(ties) > 1 and x32 != 0:
            assert c & 1 == 0, (x32, hex(c))  # ties go to the even mantissa


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 1e-2])
    x = x[np.abs(x) < 440].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_encode(v) for v in x], np.uint8)
    assert np.array_equal(got, ref)


def test_fp8_encode_saturates_and_keeps_nan():
    assert oracle.fp8_encode(449.0) == 0x7E and oracle.fp8_encode(1e30) == 0x7E
    assert oracle.fp8_encode(-float("inf")) == 0xFE
    assert oracle.fp8_encode(float("nan")) & 0x7F == 0x7F
    assert oracle.fp8_encode(-0.0) == 0x80 and oracle.fp8_encode(2.0 ** -11) == 0x00


def _fp8_case(seed, T=6, H=2, d=128, nb=5):
    g = torch.Generator().manual_seed(seed)
    key = torch.randn(T, H, d, generator=g).to(torch.bfloat16)
    value = torch.randn(T, H, d, generator=g).to(torch.bfloat16)
    slots = np.array([3, 17, -1, 40, 79, 64], np.int64)[:T]
    return key, value, slots, nb


def test_fp8_kv_write_touches_only_written_slots():
    key, value, slots, nb = _fp8_case(1)
    kc = np.full((nb, 2, 16, 128), 0x55, np.uint8)
    vc = np.full((nb, 2, 128 * 16), 0x55, np.uint8)
    oracle.kv_write_fp8(key, value, kc, vc, slots, 16, 0.75, 1.5)
    n_written = int((slots >= 0).sum()) * 2 * 128
    for pool in (kc, vc):
        changed = int((pool != 0x55).sum())
        assert n_written - 64 <= changed <= n_written  # a code may equal the filler
    # blocks no slot names are untouched
    hit = {int(s) // 16 for s in slots if s >= 0}
    for blk in range(nb):
        if blk not in hit:
            assert (kc[blk] == 0x55).all() and (vc[blk] == 0x55).all()


def test_fp8_value_row_reads_back_dequantized():
    """A one-key context returns its V row exactly: each element is
    fp8_decode(fp8_encode(v / v_scale)) * v_scale, the division in binary32."""
    key, value, _, _ = _fp8_case(6)
    ks, vs = 0.75, 1.5
    for i in range(key.shape[0]):
        kc1 = np.zeros((1, 2, 16, 128), np.uint8)
        vc1 = np.zeros((1, 2, 128 * 16), np.uint8)
        oracle.kv_write_fp8(key[i:i + 1], value[i:i + 1], kc1, vc1, [0], 16, ks, vs)
        q = torch.randn(1, 2, 128).to(torch.bfloat16)
        out = oracle.attention(q, kc1, vc1, [0, 1], [1], [[0]], 16, 1.0, kv_scales=(ks, vs))
        for h in range(2):
            v_exp = [oracle.fp8_decode(oracle.fp8_encode(np.float32(x) / np.float32(vs))) * vs
                     for x in value[i, h].float().numpy()]
            assert np.array_equal(out[0, h], np.array(v_exp))


def test_fp8_attention_equals_16bit_attention_on_dequantized_pools():
    """Attention over an FP8 pool equals attention over a bf16 pool holding
    code x scale for every element (exact in bf16 for power-of-two scales)."""
    rng = np.random.default_rng(8)
    nst, nct = [1, 5, 1, 20], [40, 3, 70, 0]
    R, H, Hq, d, bs = 4, 2, 8, 128, 16
    seq = [a + b for a, b in zip(nst, nct)]
    need = [-(-L // bs) for L in seq]
    nb = sum(need) + 3
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((R, max(need)), -1, np.int32)
    cur = 0
    for r in range(R):
        bt[r, :need[r]] = perm[cur:cur + need[r]]
        cur += need[r]
    g = torch.Generator().manual_seed(9)
    T = sum(nst)
    all_k = torch.randn(nb * bs, H, d, generator=g).to(torch.bfloat16)
    all_v = torch.randn(nb * bs, H, d, generator=g).to(torch.bfloat16)
    q = torch.randn(T, Hq, d, generator=g).to(torch.bfloat16)
    ks, vs = 0.25, 2.0
    kc8 = np.zeros((nb, H, bs, d), np.uint8)
    vc8 = np.zeros((nb, H, d * bs), np.uint8)
    slots = np.arange(nb * bs, dtype=np.int64)
    oracle.kv_write_fp8(all_k, all_v, kc8, vc8, slots, bs, ks, vs)
    deq = np.vectorize(lambda x, s: oracle.fp8_decode(oracle.fp8_encode(np.float32(x) / np.float32(s))) * s)
    kd = torch.from_numpy(deq(all_k.float().numpy(), ks).astype(np.float32)).to(torch.bfloat16)
    vd = torch.from_numpy(deq(all_v.float().numpy(), vs).astype(np.float32)).to(torch.bfloat16)
    kc16 = torch.zeros(nb, H, bs, d, dtype=torch.bfloat16)
    vc16 = torch.zeros(nb, H, d, bs, dtype=torch.bfloat16)
    oracle.kv_write(kd, vd, kc16, vc16, slots, bs)
    qsl = np.concatenate([[0], np.cumsum(nst)]).astype(np.int32)
    ref = oracle.attention(q, kc16, vc16, qsl, seq, bt, bs, 1 / math.sqrt(d))
    got = oracle.attention(q, kc8, vc8, qsl, seq, bt, bs, 1 / math.sqrt(d), kv_scales=(ks, vs))
    assert np.array_equal(got, ref)


def test_fp8_value_layout_fills_every_byte_of_a_run():
    """Writing all 16 tokens of a block touches every byte of its V run once."""
    g = torch.Generator().manual_seed(2)
    key = torch.randn(16, 1, 128, generator=g).to(torch.bfloat16) + 3.0  # no zero codes
    value = torch.randn(16, 1, 128, generator=g).to(torch.bfloat16) + 3.0
    kc = np.zeros((1, 1, 16, 128), np.uint8)
    vc = np.zeros((1, 1, 128 * 16), np.uint8)
    oracle.kv_write_fp8(key, value, kc, vc, np.arange(16), 16, 1.0, 1.0)
    assert (vc != 0).all() and (kc != 0).all()


def _fp8_distinct_codes(d):
    """Codes for dims 0..d-1 of one row, all different, none zero or NaN:
    0x01..0x7E, then negative codes."""
    pos = list(range(0x01, 0x7F))
    return np.array((pos + [0x80 | c for c in pos])[:d], np.uint8)


def test_fp8_pool_byte_positions():
    """Where one token's K and V rows land in the FP8 pools, byte by byte, for
    every token position of a block and both heads of a two-head pool, written
    out from the documented orders: each K (block, head) run ordered
    [dim / 64][token][dim % 64]; each V (block, head) run ordered
    [dim / 64][token / 4][dim % 16][(dim / 16) % 4][token % 4].  Each element
    of the row is the exact value of a distinct code (scale 1), so its byte is
    found wherever it lands."""
    H, d, bs, nb = 2, 128, 16, 3
    codes = [_fp8_distinct_codes(d), np.roll(_fp8_distinct_codes(d), 37)]
    vals = np.array([[oracle.fp8_decode(int(c)) for c in codes[h]] for h in range(H)])
    row = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16)[None]  # exact in bf16
    assert np.array_equal(row.float().numpy()[0], vals)
    filler = 0xFF  # a NaN code: no finite value encodes to it
    for tok in range(bs):
        blk = 1
        kc = np.full((nb, H, bs, d), filler, np.uint8)
        vc = np.full((nb, H, d * bs), filler, np.uint8)
        oracle.kv_write_fp8(row, row, kc, vc, [blk * bs + tok], bs, 1.0, 1.0)
        kflat, vflat = kc.reshape(-1), vc.reshape(-1)
        for h in range(H):
            run = (blk * H + h) * d * bs
            for dim in range(d):
                k_at = run + (dim // 64) * 1024 + tok * 64 + dim % 64
                v_at = run + (dim // 64) * 1024 + (tok // 4) * 256 + (dim % 16) * 16 + \
                    ((dim // 16) % 4) * 4 + tok % 4
                assert kflat[k_at] == codes[h][dim], ("K", tok, h, dim)
                assert vflat[v_at] == codes[h][dim], ("V", tok, h, dim)
        assert int((kc != filler).sum()) == H * d and int((vc != filler).sum()) == H * d


def test_fp8_write_rejects_bad_arguments():
    key, value, slots, nb = _fp8_case(5)
    kc = np.zeros((nb, 2, 16, 128), np.uint8)
    vc = np.zeros((nb, 2, 128 * 16), np.uint8)
    for ks in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(oracle.OracleError):
            oracle.kv_write_fp8(key, value, kc, vc, slots, 16, ks, 1.0)
    with pytest.raises(oracle.OracleError):
        oracle.kv_write_fp8(key, value, kc, vc, np.array([3, 3, -1, 4, 5, 6]), 16, 1.0, 1.0)


# ---------------------------------------------------------------------------
# input ids and the discard mask ("Building the Batch", "How they are
# computed"; "vLLM's Model Runner...", "The batch contains rows that must
# not be sampled")
# ---------------------------------------------------------------------------

def test_input_ids_token_indices_worked_example(golden):
    g = golden["token_indices_example"]
    M = 1000
    table = np.arange(3 * M, dtype=np.int32).reshape(3, M) * 7 + 5
    out = oracle.input_ids(table, g["req_indices"], g["positions"], [2, 5, 3], [2, 5, 3])
    want = [a * M + b for a, b in g["token_indices_in_units_of_M"]]
    assert out["token_indices"].tolist() == want
    assert out["input_ids"].tolist() == [int(table.reshape(-1)[k]) for k in want]


def test_discard_mask_worked_example(golden):
    g = golden["discard_mask_example"]
    nst, nct = g["num_scheduled_tokens"], g["num_computed_tokens"]
    prep = oracle.prepare(nst, nct, _table([[0] * 7, [1], [2] * 3]), block_size=16,
                          num_blocks=3)
    table = np.zeros((3, 700), np.int32)
    out = oracle.input_ids(table, prep["req_indices"], prep["positions"], prep["seq_lens"],
                           g["num_tokens_total"])
    assert out["discard_request_mask"].astype(bool).tolist() == g["discard_request_mask"]


def test_input_ids_gather_random_batches():
    rng = np.random.default_rng(21)
    for _ in range(20):
        R = int(rng.integers(1, 12))
        M = int(rng.integers(64, 300))
        nst = rng.integers(1, 20, R)
        nct = rng.integers(0, M - 20, R)
        total = nct + nst + rng.integers(-1, 5, R)  # some requests still mid-prompt
        table = rng.integers(0, 50000, (R, M)).astype(np.int32)
        bt = np.zeros((R, -(-M // 16)), np.int32)
        prep = oracle.prepare(nst, nct, bt, block_size=16, num_blocks=1)
        out = oracle.input_ids(table, prep["req_indices"], prep["positions"], prep["seq_lens"],
                               total)
        i = 0
        for r in range(R):  # brute force: the t-th new token of r sits at nct + t of row r
            for t in range(int(nst[r])):
                assert out["input_ids"][i] == table[r, nct[r] + t]
                i += 1
        assert out["discard_request_mask"].tolist() == [int(nct[r] + nst[r] < total[r])
                                                        for r in range(R)]


def test_input_ids_rejects_positions_outside_the_table():
    with pytest.raises(oracle.OracleError):
        oracle.input_ids(np.zeros((2, 8), np.int32), [0, 1], [3, 8], [4, 9], [4, 9])
    with pytest.raises(oracle.OracleError):
        oracle.input_ids(np.zeros((2, 8), np.int32), [0, 2], [3, 1], [4, 2], [4, 2])


# ---------------------------------------------------------------------------
# block copy-on-write and zeroing ("How vLLM Works Internally: A Deep Dive",
# "Copy-on-Write for Beam Search"; "Inside vLLM...", Part 2,
# new_block_ids_to_zero)
# ---------------------------------------------------------------------------

def test_copy_and_zero_blocks_post_state():
    rng = np.random.default_rng(2)
    kc = rng.integers(0, 256, (9, 2, 16, 64), dtype=np.uint8)
    vc = rng.integers(0, 256, (9, 2, 64, 16), dtype=np.uint8)
    k0, v0 = kc.copy(), vc.copy()
    oracle.copy_blocks(kc, vc, [[3, 7], [1, 0]])
    assert np.array_equal(kc[7], k0[3]) and np.array_equal(vc[7], v0[3])
    assert np.array_equal(kc[0], k0[1]) and np.array_equal(vc[0], v0[1])
    for b in (1, 2, 3, 4, 5, 6, 8):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])
    oracle.zero_blocks(kc, vc, [2, 8])
    assert not kc[2].any() and not vc[2].any() and not kc[8].any() and not vc[8].any()
    assert np.array_equal(kc[4], k0[4]) and np.array_equal(vc[5], v0[5])
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(kc, vc, [[0, 9]])
    with pytest.raises(oracle.OracleError):
        oracle.zero_blocks(kc, vc, [-1])


def test_copy_on_write_keeps_the_other_beam_intact():
    """Two beams share block 0 (positions 0..15) and diverge: beam 1 copies it
    to block 2, points its table there and overwrites its last slot.  Beam 0's
    attention is unchanged; beam 1 equals attention over an unshared pool that
    holds the same rows."""
    g = torch.Generator().manual_seed(4)
    H, d, bs = 2, 64, 16
    kc = torch.randn(4, H, bs, d, generator=g).to(torch.bfloat16)
    vc = torch.randn(4, H, d, bs, generator=g).to(torch.bfloat16)
    q = torch.randn(2, 4, d, generator=g).to(torch.bfloat16)
    new_k = torch.randn(1, H, d, generator=g).to(torch.bfloat16)
    new_v = torch.randn(1, H, d, generator=g).to(torch.bfloat16)
    qsl, sl = [0, 1, 2], [16, 16]
    before = oracle.attention(q, kc, vc, qsl, sl, [[0], [0]], bs, 0.125)
    oracle.copy_blocks(kc, vc, [[0, 2]])
    oracle.kv_write(new_k, new_v, kc, vc, [2 * bs + 15], bs)  # beam 1 writes its own copy
    after = oracle.attention(q, kc, vc, qsl, sl, [[0], [2]], bs, 0.125)
    assert np.array_equal(after[0], before[0])
    fresh_k, fresh_v = kc[[0]].clone(), vc[[0]].clone()
    oracle.kv_write(new_k, new_v, fresh_k, fresh_v, [15], bs)
    alone = oracle.attention(q[1:], fresh_k, fresh_v, [0, 1], [16], [[0]], bs, 0.125)
    assert np.array_equal(after[1], alone[0])
