"""Shared helpers of the GPU parity tests: run one step of the hot path through
the C ABI and the same step through the fp64 oracle, on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_prepare_amd as pkv

BF16_MAX_ABS = 2e-2
BF16_REL_FRO = 1e-2
F32_MAX_ABS = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def gpu_prepare(wl, qsl_len=None):
    dev = wl.q.device
    nst = torch.from_numpy(wl.num_scheduled_tokens).to(dev)
    nct = torch.from_numpy(wl.num_computed_tokens).to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    out = pkv.prepare_inputs(nst, nct, bt, num_tokens=wl.num_tokens, block_size=wl.block_size,
                             num_blocks=wl.num_blocks, qsl_len=qsl_len)
    return out, bt


def gpu_scales(wl):
    """One-element float32 device tensors of an FP8 workload's scales (else None, None)."""
    if wl.kv_scales is None:
        return None, None
    dev = wl.q.device
    return (torch.tensor([wl.kv_scales[0]], dtype=torch.float32, device=dev),
            torch.tensor([wl.kv_scales[1]], dtype=torch.float32, device=dev))


def gpu_step(wl, split_tokens=0):
    """prepare -> kv_write -> attention on the GPU (pool copies are written).

    The output and the attention workspace are filled with NaN (0xFF bytes)
    beforehand, and every output row must come back finite: a row, tile or
    partition that no kernel wrote (or that read a partial nobody wrote)
    shows up here even where the oracle comparison samples rows."""
    prep, bt = gpu_prepare(wl)
    kc, vc = wl.key_cache.clone(), wl.value_cache.clone()
    ks, vs = gpu_scales(wl)
    if ks is None:
        pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"],
                           block_size=wl.block_size)
    else:
        pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], ks, vs,
                               block_size=wl.block_size)
    out = torch.full_like(wl.q, float("nan"))
    need = pkv.attention_workspace_bytes(wl.num_reqs, wl.num_tokens, wl.num_q_heads,
                                         wl.num_kv_heads, wl.head_dim, wl.max_query_len,
                                         wl.max_seq_len, split_tokens, wl.dtype)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=wl.q.device)
    pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], bt,
                        max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                        scale=wl.scale, split_tokens=split_tokens, k_scale=ks, v_scale=vs,
                        out=out, workspace=ws)
    torch.cuda.synchronize()
    bad = (~torch.isfinite(out)).reshape(out.shape[0], -1).any(1).nonzero()
    assert bad.numel() == 0, \
        f"{wl.name}: {bad.numel()} output rows not finite, first {bad[:8].flatten().tolist()}"
    return prep, kc, vc, out


def oracle_step(wl, rows=None):
    """The same step through the oracle, from the generator's (pre-write) inputs."""
    prep = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                          wl.block_size, wl.num_blocks)
    kc, vc = wl.key_cache.cpu().clone(), wl.value_cache.cpu().clone()
    if wl.kv_scales is None:
        oracle.kv_write(wl.key.cpu(), wl.value.cpu(), kc, vc, prep["slot_mapping"],
                        wl.block_size)
    else:
        oracle.kv_write_fp8(wl.key.cpu(), wl.value.cpu(), kc, vc, prep["slot_mapping"],
                            wl.block_size, *wl.kv_scales)
    ref = oracle.attention(wl.q.cpu(), kc, vc, prep["query_start_loc"], prep["seq_lens"],
                           wl.block_table, wl.block_size, wl.scale, rows=rows,
                           kv_scales=wl.kv_scales)
    return prep, kc, vc, ref


def bits_view(t):
    if t.element_size() == 1:
        return t.view(torch.uint8)
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def assert_prepare_equal(got, ref, what=""):
    for k, v in ref.items():
        g = got[k].cpu().numpy()
        assert g.dtype == v.dtype, f"{what} {k}: dtype {g.dtype} vs {v.dtype}"
        assert np.array_equal(g, v), f"{what} {k} differs: first mismatch at " \
            f"{int(np.argmax(g != v)) if g.shape == v.shape else 'shape'}"


def attention_errors(got, ref):
    g = got.double().cpu().numpy()
    diff = g - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else 0.0
    return max_abs, rel, bool(np.isfinite(g).all())


def assert_attention_close(got, ref, dtype, what=""):
    max_abs, rel, finite = attention_errors(got, ref)
    log(f"  {what}: max_abs={max_abs:.3e} rel_fro={rel:.3e}")
    assert finite, f"{what}: non-finite output"
    if dtype == torch.float32:
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs {max_abs}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max abs {max_abs}"
        assert rel <= BF16_REL_FRO, f"{what}: rel fro {rel}"
