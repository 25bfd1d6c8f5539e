"""GPU parity of pkv_prepare_inputs and pkv_kv_cache_write against the oracle
(bit-exact), through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import assert_prepare_equal, bits_view, device, gpu_prepare, log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "prepare_page_examples.json")


def _table(rows):
    width = max(len(r) for r in rows)
    t = np.full((len(rows), width), -1, np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    return t


def run_prepare(nst, nct, bt, bs, nb, qsl_len=None, num_tokens=None):
    dev = device()
    nst = np.asarray(nst, np.int32)
    nct = np.asarray(nct, np.int32)
    T = int(nst.sum()) if num_tokens is None else num_tokens
    return pkv.prepare_inputs(torch.from_numpy(nst).to(dev), torch.from_numpy(nct).to(dev),
                              torch.from_numpy(np.ascontiguousarray(bt)).to(dev), num_tokens=T,
                              block_size=bs, num_blocks=nb, qsl_len=qsl_len)


def test_prepare_page_examples():
    g = json.load(open(GOLDEN))
    e = g["worked_example_253"]
    out = run_prepare(e["num_scheduled_tokens"], [0, 0, 0], _table([[0], [1], [2]]), 16, 3)
    assert out["req_indices"].tolist() == e["req_indices"]
    assert out["positions"].tolist() == e["query_pos"]
    assert out["query_start_loc"].tolist() == e["query_start_loc"]
    assert out["logits_indices"].tolist() == e["logits_indices"]
    e = g["packed_batch_411"]
    out = run_prepare(e["num_scheduled_tokens"], e["num_computed_tokens"],
                      _table([[0], [1, 2, 3, 4], [5, 6]]), 16, 8)
    assert out["positions"].tolist() == e["positions"]
    assert out["query_start_loc"].tolist() == e["query_start_loc"]
    e = g["go_program_bs4"]
    out = run_prepare(e["num_scheduled_tokens"], e["num_computed_tokens"],
                      _table(e["block_tables"]), e["block_size"], 16)
    rows_b = (out["req_indices"] == 1).nonzero().flatten()
    assert out["slot_mapping"][rows_b].tolist() == e["request_B_slots"]
    e = g["nano_block_mapping"]
    out = run_prepare([10], [0], _table([e["block_table"]]), e["block_size"], 16)
    assert (out["slot_mapping"] // 4).tolist() == e["token_physical_block"]


@pytest.mark.parametrize("seed", range(8))
def test_prepare_random_vs_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.choice([1, 5, 255, 256, 257, 700]))
    bs = int(rng.choice([1, 4, 16]))
    nst = rng.integers(0, 12, size=R).astype(np.int32)
    nst[rng.random(R) < 0.2] = 0
    if seed % 2:
        nst[rng.integers(0, R)] = 1500   # one long chunk: rows span several workgroups
    nct = rng.integers(0, 300, size=R).astype(np.int32)
    need = (nst + nct + bs - 1) // bs
    nb = int(need.sum()) + 7
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((R, int(need.max()) + 3), -1, np.int32)
    c = 0
    for r in range(R):
        bt[r, :need[r]] = perm[c:c + need[r]]
        c += need[r]
    qsl_len = R + 1 + int(rng.integers(0, 40))
    got = run_prepare(nst, nct, bt, bs, nb, qsl_len=qsl_len)
    ref = oracle.prepare(nst, nct, bt, bs, nb, qsl_len=qsl_len)
    log(f"  R={R} T={int(nst.sum())} bs={bs}")
    assert_prepare_equal(got, ref, f"seed {seed}")


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_prepare_configs(idx):
    s = workloads.config_structure(idx)
    wl = workloads.build(f"cfg{idx}-structure", s["num_scheduled_tokens"],
                         s["num_computed_tokens"], num_q_heads=1, num_kv_heads=1, head_dim=8,
                         seed=1000 + idx, device=device())
    got, _ = gpu_prepare(wl)
    ref = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                         wl.block_size, wl.num_blocks)
    assert_prepare_equal(got, ref, f"config {idx}")


def test_prepare_edge_cases():
    # empty batch: only query_start_loc is written
    out = run_prepare(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, 1), np.int32),
                      16, 1, qsl_len=5)
    assert out["query_start_loc"].tolist() == [0] * 5
    # requests with no tokens at the start, middle and end
    nst, nct = [0, 3, 0, 0, 2, 0], [5, 1, 9, 0, 30, 2]
    bt = _table([[0], [1], [2], [3], [4, 5], [6]])
    assert_prepare_equal(run_prepare(nst, nct, bt, 16, 8, qsl_len=9),
                         oracle.prepare(nst, nct, bt, 16, 8, qsl_len=9), "zero-length")
    # block id outside the pool, and a position past the table width -> slot -1
    out = run_prepare([2, 2], [0, 15], _table([[9], [1]]), 16, 4)
    assert out["slot_mapping"].tolist() == [-1, -1, 31, -1]
    # host token count larger than the device sum -> trailing rows are -1
    out = run_prepare([2, 1], [0, 0], _table([[0], [1]]), 16, 4, num_tokens=5)
    assert out["req_indices"].tolist() == [0, 0, 1, -1, -1]
    assert out["slot_mapping"].tolist() == [0, 1, 16, -1, -1]


# ---------------------------------------------------------------------------
# kv_write
# ---------------------------------------------------------------------------

def _kv_case(T, H, d, bs, nb, dtype, seed, consecutive):
    g = torch.Generator(device="cpu").manual_seed(seed)
    rng = np.random.default_rng(seed)
    key = torch.randn(T, H, d, generator=g).to(dtype)
    val = torch.randn(T, H, d, generator=g).to(dtype)
    kc = torch.randn(nb, H, d * bs, generator=g).to(dtype)
    vc = torch.randn(nb, H, d * bs, generator=g).to(dtype)
    if consecutive:  # a prompt chunk: runs of consecutive slots, some not block aligned
        start = int(rng.integers(0, nb * bs - T))
        slots = np.arange(start, start + T, dtype=np.int64)
    else:
        slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.1] = -1          # padding rows
    if T > 3:
        slots[2] = nb * bs + 5               # past the pool: skipped
    return key, val, kc, vc, slots


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128, 96, 40])   # 96: three K slabs; 40: plain K and V runs
@pytest.mark.parametrize("bs", [16, 4, 5])
@pytest.mark.parametrize("consecutive", [False, True])
def test_kv_write_vs_oracle(dtype, d, bs, consecutive):
    T, H = 77, 3
    nb = 40 if bs == 16 else 160
    key, val, kc, vc, slots = _kv_case(T, H, d, bs, nb, dtype, 7 + d + bs, consecutive)
    okc, ovc = kc.clone(), vc.clone()
    oslots = slots.copy()
    oslots[oslots >= nb * bs] = -1          # the oracle rejects what the kernel skips
    oracle.kv_write(key, val, okc, ovc, oslots, bs)
    dev = device()
    gkc, gvc = kc.to(dev), vc.to(dev)
    pkv.kv_cache_write(key.to(dev), val.to(dev), gkc, gvc, torch.from_numpy(slots).to(dev),
                       block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(bits_view(gkc.cpu()), bits_view(okc))
    assert torch.equal(bits_view(gvc.cpu()), bits_view(ovc))


def test_kv_write_strided_rows():
    """K and V as views into one fused [T, (Hq + 2 Hkv) * d] projection output."""
    T, Hq, H, d, bs, nb = 50, 8, 2, 128, 16, 12
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(3)
    qkv = torch.randn(T, (Hq + 2 * H) * d, generator=g).to(torch.bfloat16)
    key = qkv[:, Hq * d:(Hq + H) * d].view(T, H, d)
    val = qkv[:, (Hq + H) * d:].view(T, H, d)
    kc = torch.zeros(nb, H, d * bs, dtype=torch.bfloat16)
    vc = torch.zeros(nb, H, d * bs, dtype=torch.bfloat16)
    slots = np.random.default_rng(4).permutation(nb * bs)[:T].astype(np.int64)
    okc, ovc = kc.clone(), vc.clone()
    oracle.kv_write(key.contiguous(), val.contiguous(), okc, ovc, slots, bs)
    gqkv = qkv.to(dev)
    gkc, gvc = kc.to(dev), vc.to(dev)
    pkv.kv_cache_write(gqkv[:, Hq * d:(Hq + H) * d].view(T, H, d),
                       gqkv[:, (Hq + H) * d:].view(T, H, d), gkc, gvc,
                       torch.from_numpy(slots).to(dev), block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(bits_view(gkc.cpu()), bits_view(okc))
    assert torch.equal(bits_view(gvc.cpu()), bits_view(ovc))


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_kv_write_configs(idx):
    wl = workloads.config(idx, device=device())
    prep, _ = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"], block_size=wl.block_size)
    torch.cuda.synchronize()
    ref = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                         wl.block_size, wl.num_blocks)
    okc, ovc = wl.key_cache.cpu(), wl.value_cache.cpu()
    oracle.kv_write(wl.key.cpu(), wl.value.cpu(), okc, ovc, ref["slot_mapping"], wl.block_size)
    assert torch.equal(bits_view(kc.cpu()), bits_view(okc)), "K pool"
    assert torch.equal(bits_view(vc.cpu()), bits_view(ovc)), "V pool"


# ---------------------------------------------------------------------------
# FP8 cache write: E4M3 codes of value / scale must match the oracle byte
# for byte (the quantised code is an integer decision taken in binary32 on
# both sides).
# ---------------------------------------------------------------------------

def _fp8_scales(dev, ks, vs):
    return (torch.tensor([ks], dtype=torch.float32, device=dev),
            torch.tensor([vs], dtype=torch.float32, device=dev))


def test_kv_write_fp8_rounding_matches_oracle():
    """Every E4M3 value, every midpoint between neighbours (ties), values just
    off the midpoints, subnormals, saturation and zeros, through the kernel's
    conversion with scale 1, against the oracle's encoder."""
    table = np.array([oracle.fp8_decode(c) for c in range(256)])
    pos = np.unique(np.abs(table[~np.isnan(table)]))
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                           [447.9, 448.0, 460.0, 464.0, 470.0, 1e6, 2.0 ** -10, 2.0 ** -11, 0.0]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    d = 128
    T = -(-len(vals) // d)
    flat = np.zeros(T * d, np.float32)
    flat[:len(vals)] = vals
    key = torch.from_numpy(flat.reshape(T, 1, d))
    val = key.clone()
    dev = device()
    nb = -(-T // 16)
    kc = torch.zeros(nb, 1, d * 16, dtype=torch.uint8, device=dev)
    vc = torch.zeros(nb, 1, d * 16, dtype=torch.uint8, device=dev)
    ks, vs = _fp8_scales(dev, 1.0, 1.0)
    pkv.kv_cache_write_fp8(key.to(dev), val.to(dev), kc, vc, torch.arange(T, device=dev), ks, vs,
                           block_size=16)
    torch.cuda.synchronize()
    # K runs are [dim / 64][token][dim % 64]: back to token-major order
    got = kc.cpu().reshape(nb, 1, d // 64, 16, 64).permute(0, 1, 3, 2, 4).reshape(-1).numpy()
    got = got[:len(vals)]
    want = np.array([oracle.fp8_encode(v) for v in vals], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("consecutive", [False, True])
def test_kv_write_fp8_vs_oracle(dtype, d, consecutive):
    T, H, nb, bs = 77, 3, 40, 16
    key, val, _, _, slots = _kv_case(T, H, d, bs, nb, dtype, 11 + d, consecutive)
    key, val = key * 3, val * 0.5
    g = torch.Generator().manual_seed(d)
    kc = torch.randint(0, 256, (nb, H, d * bs), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (nb, H, d * bs), generator=g, dtype=torch.uint8)
    okc, ovc = kc.clone(), vc.clone()
    oslots = slots.copy()
    oslots[oslots >= nb * bs] = -1
    oracle.kv_write_fp8(key, val, okc, ovc, oslots, bs, 0.37, 2.5)
    dev = device()
    gkc, gvc = kc.to(dev), vc.to(dev)
    ks, vs = _fp8_scales(dev, 0.37, 2.5)
    pkv.kv_cache_write_fp8(key.to(dev), val.to(dev), gkc, gvc, torch.from_numpy(slots).to(dev),
                           ks, vs, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(gkc.cpu(), okc)
    assert torch.equal(gvc.cpu(), ovc)
