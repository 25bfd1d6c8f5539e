"""GPU parity of the FP8 KV cache ("How vLLM Works Internally: A Deep Dive",
"FP8 KV Cache"; the write call's kv_cache_dtype / k_scale / v_scale in "Inside
vLLM: Following One Request from the API to GPU Execution", Part 5): prepare ->
pkv_kv_cache_write_fp8 -> pkv_paged_attention_varlen_fp8 through the C ABI
against the oracle on the same FP8 pools.  Pools must match byte for byte;
attention within the bf16 bar (the oracle reads every code exactly, so the
comparison measures the kernels' arithmetic, not the quantisation)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_prepare_amd import workloads

from gpu_helpers import (assert_attention_close, assert_prepare_equal, device, gpu_step, log,
                         oracle_step)
from test_gpu_b_attention import SMALL, sample_rows

pytestmark = pytest.mark.gpu

SCALES = (0.0125, 0.02)


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_fp8_attention_small(case):
    nst, nct, Hq, Hkv, d = SMALL[case]
    wl = workloads.build(f"small{case}", nst, nct, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                         seed=150 + case, device=device(), pool_slack=1.3, extra_table_cols=2)
    wl = workloads.to_fp8(wl, *SCALES)
    prep, kc, vc, out = gpu_step(wl)
    ref_prep, okc, ovc, ref = oracle_step(wl)
    assert torch.equal(kc.cpu(), okc), "K pool"
    assert torch.equal(vc.cpu(), ovc), "V pool"
    assert_attention_close(out, ref, wl.dtype, f"fp8 small{case}")


@pytest.mark.parametrize("split_tokens", [32, 96, 0])
def test_fp8_attention_partitions(split_tokens):
    wl = workloads.build("fp8split", [1, 1, 1, 2, 1, 40], [2000, 31, 700, 901, 129, 300],
                         num_q_heads=32, num_kv_heads=8, head_dim=128, seed=78, device=device(),
                         pool_slack=1.1)
    wl = workloads.to_fp8(wl, 0.05, 0.03)
    _, _, _, out = gpu_step(wl, split_tokens=split_tokens)
    _, _, _, ref = oracle_step(wl)
    assert_attention_close(out, ref, wl.dtype, f"fp8 split {split_tokens}")


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_fp8_attention_config(idx):
    """The named configurations with FP8 pools, in the launch configuration the
    benchmark times (sampled rows; every pool byte compared)."""
    log(f"config {idx} fp8: {workloads.CONFIG_NAMES[idx]}")
    wl = workloads.to_fp8(workloads.config(idx, device=device()), *SCALES)
    prep, kc, vc, out = gpu_step(wl)
    rows = sample_rows(wl)
    ref_prep, okc, ovc, ref = oracle_step(wl, rows=rows)
    assert_prepare_equal(prep, ref_prep, f"config {idx}")
    assert torch.equal(kc.cpu(), okc), "K pool"
    assert torch.equal(vc.cpu(), ovc), "V pool"
    got = out if rows is None else out[torch.from_numpy(rows).long().to(out.device)]
    assert_attention_close(got, ref, wl.dtype, f"config {idx} fp8")


def test_fp8_scale_is_applied_to_keys_and_values():
    """Over the same written pools: doubling v_scale doubles the output exactly;
    another k_scale gives the oracle's result for that scale."""
    import oracle
    import paged_kv_cache_prepare_amd as pkv
    from gpu_helpers import gpu_prepare, gpu_scales
    dev = device()
    wl = workloads.to_fp8(workloads.build("sc", [1, 20], [300, 40], num_q_heads=8,
                                          num_kv_heads=2, head_dim=128, seed=3, device=dev),
                          0.02, 0.02)
    prep, bt = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    ks, vs = gpu_scales(wl)
    pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], ks, vs, block_size=16)

    def attend(k_scale, v_scale):
        out = pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                                  max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                                  scale=wl.scale, k_scale=torch.tensor([k_scale], device=dev),
                                  v_scale=torch.tensor([v_scale], device=dev))
        torch.cuda.synchronize()
        return out

    base, twice = attend(0.02, 0.02), attend(0.02, 0.04)
    assert torch.equal(twice.float(), 2 * base.float())
    out3 = attend(0.03, 0.02)
    ref3 = oracle.attention(wl.q.cpu(), kc.cpu(), vc.cpu(), prep["query_start_loc"].cpu(),
                            prep["seq_lens"].cpu(), wl.block_table, 16, wl.scale,
                            kv_scales=(0.03, 0.02))
    assert_attention_close(out3, ref3, wl.dtype, "k_scale 0.03")


def test_fp8_attention_prompt_rows():
    """Configuration 4's prompt rows alone over FP8 pools (1256 tiles on the
    two-per-CU resident prefill workgroups), sampled rows."""
    wl = workloads.config(4, device=device())
    group = wl.num_q_heads // wl.num_kv_heads
    wl = workloads.select(wl, np.nonzero(wl.num_scheduled_tokens * group > 16)[0])
    wl = workloads.to_fp8(wl, *SCALES)
    prep, kc, vc, out = gpu_step(wl)
    rows = sample_rows(wl)
    _, _, _, ref = oracle_step(wl, rows=rows)
    got = out if rows is None else out[torch.from_numpy(rows).long().to(out.device)]
    assert_attention_close(got, ref, wl.dtype, "config 4 prompt rows fp8")
