"""The checked build (libpkv_checked.so): on valid device data it returns
exactly what the regular build returns (same kernels); on device data that
breaks a documented precondition it returns PKV_ERR_DEVICE_DATA, names the
failed check, and launches nothing else (outputs keep their sentinels).
Every bad input here is one the validation kernel reads safely; the regular
kernels never see it."""
import numpy as np
import pytest
import torch

import paged_kv_cache_prepare_amd as pkv
from paged_kv_cache_prepare_amd import binding, workloads

from gpu_helpers import bits_view, device, gpu_step, log

pytestmark = pytest.mark.gpu


@pytest.fixture
def checked():
    binding.use_checked(True)
    assert binding.load().pkv_debug_checks_enabled() == 1
    yield
    binding.use_checked(False)


def _fails(check, fn, *args, **kw):
    with pytest.raises(pkv.PkvError) as e:
        fn(*args, **kw)
    assert e.value.status == binding.ERR_DEVICE_DATA, str(e.value)
    assert check in binding.check_flags(), (check, binding.check_flags())


def _i32(a):
    return torch.tensor(np.asarray(a, np.int32), device=device())


def _small():
    return workloads.build("chk", [1, 5, 1], [40, 0, 300], num_q_heads=8, num_kv_heads=2,
                           head_dim=128, seed=12, device=device(), pool_slack=1.3,
                           extra_table_cols=1)


def test_checked_build_matches_regular_on_valid_data():
    wl = _small()
    binding.use_checked(False)
    ref = gpu_step(wl, split_tokens=64)
    binding.use_checked(True)
    try:
        got = gpu_step(wl, split_tokens=64)
    finally:
        binding.use_checked(False)
    for k in ref[0]:
        assert torch.equal(got[0][k], ref[0][k]), k
    for a, b in zip(got[1:], ref[1:]):
        assert torch.equal(bits_view(a), bits_view(b))


def test_prepare_checks(checked):
    wl = _small()
    bt = torch.from_numpy(wl.block_table).to(device())
    nct = torch.from_numpy(wl.num_computed_tokens).to(device())
    kw = dict(block_size=16, num_blocks=wl.num_blocks)
    _fails("counts", pkv.prepare_inputs, _i32([1, -5, 1]), nct, bt, num_tokens=7, **kw)
    _fails("counts", pkv.prepare_inputs, _i32([1, 5, 1]), nct, bt, num_tokens=9, **kw)
    bad = bt.clone()
    bad[2, 300 // 16] = wl.num_blocks + 4      # the block request 2's new token writes to
    _fails("block_id", pkv.prepare_inputs, _i32([1, 5, 1]), nct, bad, num_tokens=7, **kw)
    narrow = bt[:, :2].contiguous()            # request 2 needs column 18
    _fails("block_id", pkv.prepare_inputs, _i32([1, 5, 1]), nct, narrow, num_tokens=7, **kw)


def test_fused_prepare_and_plan_checks(checked):
    """The checked build runs pkv_prepare_inputs_and_plan as its two calls,
    each with its device-data checks: bad prepare inputs fail before the plan,
    and valid ones give the regular build's index tensors and list header."""
    wl = _small()
    bt = torch.from_numpy(wl.block_table).to(device())
    nct = torch.from_numpy(wl.num_computed_tokens).to(device())
    kw = dict(block_size=16, num_blocks=wl.num_blocks, num_q_heads=8, num_kv_heads=2,
              head_dim=128, max_query_len=5, max_seq_len=301, split_tokens=64)
    _fails("counts", pkv.prepare_inputs_and_plan, _i32([1, -5, 1]), nct, bt, num_tokens=7, **kw)
    bad = bt.clone()
    bad[2, 300 // 16] = wl.num_blocks + 4
    _fails("block_id", pkv.prepare_inputs_and_plan, _i32([1, 5, 1]), nct, bad, num_tokens=7, **kw)
    got, ws = pkv.prepare_inputs_and_plan(_i32([1, 5, 1]), nct, bt, num_tokens=7, **kw)
    binding.use_checked(False)
    ref, ws_ref = pkv.prepare_inputs_and_plan(_i32([1, 5, 1]), nct, bt, num_tokens=7, **kw)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    words = [0, 1, 2, 4]
    assert ws[:256].view(torch.int32)[words].tolist() == ws_ref[:256].view(torch.int32)[words].tolist()


def test_write_checks(checked):
    wl = _small()
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    nslots = wl.num_blocks * 16
    _fails("slot", pkv.kv_cache_write, wl.key, wl.value, kc, vc,
           torch.tensor([5, nslots, 7, 8, 9, 10, 11], device=device()), block_size=16)
    _fails("slot_dup", pkv.kv_cache_write, wl.key, wl.value, kc, vc,
           torch.tensor([5, 6, 7, 8, 9, 10, 6], device=device()), block_size=16)
    assert torch.equal(bits_view(kc), bits_view(wl.key_cache))   # nothing was written
    f8 = workloads.to_fp8(wl, 0.0125, 0.0125)
    k8, v8 = f8.key_cache.clone(), f8.value_cache.clone()
    zero = torch.zeros(1, dtype=torch.float32, device=device())
    one = torch.ones(1, dtype=torch.float32, device=device())
    _fails("scale", pkv.kv_cache_write_fp8, wl.key, wl.value, k8, v8,
           torch.arange(7, device=device()), zero, one, block_size=16)


def test_attention_checks(checked):
    wl = _small()
    bt = torch.from_numpy(wl.block_table).to(device())
    out = torch.full_like(wl.q, float("nan"))
    kw = dict(max_query_len=5, max_seq_len=301, scale=wl.scale, out=out)
    qsl, sl = _i32([0, 1, 6, 7]), _i32([41, 5, 301])
    _fails("qsl", pkv.paged_attention, wl.q, wl.key_cache, wl.value_cache, _i32([0, 4, 2, 7]),
           sl, bt, **kw)
    _fails("lengths", pkv.paged_attention, wl.q, wl.key_cache, wl.value_cache, qsl,
           _i32([41, 3, 301]), bt, **kw)                      # q_len 5 > seq_len 3
    _fails("lengths", pkv.paged_attention, wl.q, wl.key_cache, wl.value_cache, qsl,
           _i32([41, 5, 400]), bt, **kw)                      # seq_len > max_seq_len
    bad = bt.clone()
    bad[2, 7] = -3
    _fails("block_id", pkv.paged_attention, wl.q, wl.key_cache, wl.value_cache, qsl, sl, bad,
           **kw)
    assert torch.isnan(out).all()                            # attention never ran
    log("  attention checks reported, nothing launched")


def test_input_id_and_block_list_checks(checked):
    table = torch.zeros((3, 64), dtype=torch.int32, device=device())
    sl, tot = _i32([2, 1, 1]), _i32([2, 1, 1])
    _fails("row", pkv.prepare_input_ids, table, _i32([0, 0, 3, 2]), _i32([0, 1, 0, 0]), sl, tot)
    _fails("row", pkv.prepare_input_ids, table, _i32([0, 0, 1, 2]), _i32([0, 64, 0, 0]), sl, tot)
    got = pkv.prepare_input_ids(table, _i32([0, 0, 1, -1]), _i32([0, 1, 0, -1]), sl, tot)
    assert got["input_ids"].tolist() == [0, 0, 0, -1]        # a padding row is valid
    kc = torch.zeros((8, 1024), dtype=torch.uint8, device=device())
    vc = torch.zeros_like(kc)
    _fails("pairs", pkv.copy_blocks, kc, vc, _i32([[0, 3], [1, 3]]))
    _fails("pairs", pkv.copy_blocks, kc, vc, _i32([[0, 3], [3, 4]]))
    _fails("block_id", pkv.copy_blocks, kc, vc, _i32([[0, 8]]))
    _fails("block_id", pkv.zero_blocks, kc, vc, _i32([2, -1]))
    pkv.copy_blocks(kc, vc, _i32([[0, 3], [0, 4]]))           # one source to two blocks
    pkv.zero_blocks(kc, vc, _i32([5, 5]))
    torch.cuda.synchronize()
