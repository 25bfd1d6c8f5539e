"""Thin ctypes binding over libpkv.so (include/pkv.h).

Argument marshalling only: tensors are passed as device pointers, sizes as
host integers, and the current torch stream as the HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no Python or CPU
fallback.  If the library is not built this module raises.

With the environment variable PKV_DEBUG_CHECKS=1 (or after ``use_checked()``)
the checked build libpkv_checked.so is loaded instead: same entry points, plus
device-side validation of every call's device data (it synchronises).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
REGULAR_LIB_PATH = os.path.join(HERE, "libpkv.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libpkv_checked.so")
LIB_PATH = CHECKED_LIB_PATH if os.environ.get("PKV_DEBUG_CHECKS") == "1" else REGULAR_LIB_PATH

(OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH, ERR_DEVICE_DATA,
 ERR_SCRATCH_LIMIT) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20  # PKV_NOALLOC_SCRATCH_BYTES
# PKV_CHECK_* bits of the checked build (include/pkv.h)
CHECK_BITS = {"counts": 0x001, "block_id": 0x002, "slot": 0x004, "slot_dup": 0x008, "qsl": 0x010,
              "lengths": 0x020, "row": 0x040, "pairs": 0x080, "scale": 0x100, "plan": 0x200}
F32, BF16 = 0, 1
EXPORTS = ("pkv_status_string", "pkv_debug_checks_enabled", "pkv_debug_check_flags",
           "pkv_prepare_inputs", "pkv_prepare_input_ids",
           "pkv_kv_cache_write", "pkv_kv_cache_write_fp8", "pkv_paged_attention_workspace_bytes",
           "pkv_paged_attention_varlen", "pkv_paged_attention_varlen_fp8",
           "pkv_paged_attention_plan", "pkv_paged_attention_run", "pkv_prepare_inputs_and_plan",
           "pkv_paged_attention_varlen_noalloc", "pkv_copy_blocks", "pkv_zero_blocks")


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_debug_checks_enabled.argtypes = []
    lib.pkv_debug_checks_enabled.restype = ctypes.c_int32
    lib.pkv_debug_check_flags.argtypes = []
    lib.pkv_debug_check_flags.restype = ctypes.c_uint32
    lib.pkv_prepare_inputs.argtypes = [P, P, P, i64, i32, i32, i32, i32, i64, P, P, P, P, P, P, P]
    lib.pkv_prepare_inputs.restype = ctypes.c_int
    lib.pkv_prepare_input_ids.argtypes = [P, i64, i32, P, P, i32, P, P, P, P, P, P]
    lib.pkv_prepare_input_ids.restype = ctypes.c_int
    lib.pkv_copy_blocks.argtypes = [P, P, i64, i64, P, i32, P]
    lib.pkv_copy_blocks.restype = ctypes.c_int
    lib.pkv_zero_blocks.argtypes = [P, P, i64, i64, P, i32, P]
    lib.pkv_zero_blocks.restype = ctypes.c_int
    lib.pkv_kv_cache_write.argtypes = [P, P, i64, i64, P, P, i64, P, i32, i32, i32, i32,
                                       ctypes.c_int, P]
    lib.pkv_kv_cache_write.restype = ctypes.c_int
    lib.pkv_kv_cache_write_fp8.argtypes = [P, P, i64, i64, P, P, i64, P, i32, i32, i32, i32,
                                           ctypes.c_int, P, P, P]
    lib.pkv_kv_cache_write_fp8.restype = ctypes.c_int
    lib.pkv_paged_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                                        ctypes.c_int]
    lib.pkv_paged_attention_workspace_bytes.restype = sz
    lib.pkv_paged_attention_varlen.argtypes = [P, i64, P, P, i64, P, i64, P, P, P, i64, i32, i32,
                                               i32, i32, i32, i32, i32, i32, f32, ctypes.c_int,
                                               i32, P, sz, P]
    lib.pkv_paged_attention_varlen.restype = ctypes.c_int
    lib.pkv_paged_attention_varlen_fp8.argtypes = [P, i64, P, P, i64, P, i64, P, P, P, i64, i32,
                                                   i32, i32, i32, i32, i32, i32, i32, f32, P, P,
                                                   i32, P, sz, P]
    lib.pkv_paged_attention_varlen_fp8.restype = ctypes.c_int
    lib.pkv_paged_attention_plan.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, ctypes.c_int,
                                             i32, P, sz, P]
    lib.pkv_paged_attention_plan.restype = ctypes.c_int
    lib.pkv_prepare_inputs_and_plan.argtypes = [P, P, P, i64, i32, i32, i32, i32, i64, P, P, P, P,
                                                P, P, i32, i32, i32, i32, i32, ctypes.c_int, i32,
                                                P, sz, P]
    lib.pkv_prepare_inputs_and_plan.restype = ctypes.c_int
    lib.pkv_paged_attention_run.argtypes = [P, i64, P, P, i64, P, i64, P, P, P, i64, i32, i32, i32,
                                            i32, i32, i32, i32, i32, f32, ctypes.c_int, P, P, i32,
                                            P, sz, P]
    lib.pkv_paged_attention_run.restype = ctypes.c_int
    lib.pkv_paged_attention_varlen_noalloc.argtypes = [P, i64, P, P, i64, P, i64, P, P, P, i64,
                                                       i32, i32, i32, i32, i32, i32, i32, i32,
                                                       f32, ctypes.c_int, i32, P]
    lib.pkv_paged_attention_varlen_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def use_checked(checked: bool = True) -> ctypes.CDLL:
    """Switch this process to the checked (or back to the regular) build."""
    global _lib, LIB_PATH
    LIB_PATH = CHECKED_LIB_PATH if checked else REGULAR_LIB_PATH
    _lib = None
    return load()


def check_flags() -> list[str]:
    """Names of the checks the last PKV_ERR_DEVICE_DATA call failed (checked build)."""
    bits = int(load().pkv_debug_check_flags())
    return [name for name, bit in CHECK_BITS.items() if bits & bit]


def status_string(status: int) -> str:
    return load().pkv_status_string(int(status)).decode()


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dtype}")


def _dev(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr() if t.numel() else None


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, what: str):
    if status == ERR_DEVICE_DATA:
        raise PkvError(status, f"{what} (failed checks: {', '.join(check_flags())})")
    if status != OK:
        raise PkvError(status, what)


def prepare_inputs(num_scheduled_tokens: torch.Tensor, num_computed_tokens: torch.Tensor,
                   block_table: torch.Tensor, *, num_tokens: int, block_size: int,
                   num_blocks: int, qsl_len: int | None = None, out: dict | None = None) -> dict:
    """pkv_prepare_inputs.  ``num_tokens`` is the host-side token total."""
    R = int(num_scheduled_tokens.shape[0])
    dev = num_scheduled_tokens.device
    qsl_len = R + 1 if qsl_len is None else int(qsl_len)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"req_indices": torch.empty(num_tokens, **i32),
               "positions": torch.empty(num_tokens, **i32),
               "slot_mapping": torch.empty(num_tokens, dtype=torch.int64, device=dev),
               "query_start_loc": torch.empty(qsl_len, **i32),
               "seq_lens": torch.empty(R, **i32),
               "logits_indices": torch.empty(R, **i32)}
    assert block_table.dim() == 2 and (block_table.numel() == 0 or block_table.stride(1) == 1)
    st = load().pkv_prepare_inputs(
        _dev(num_scheduled_tokens, torch.int32, "num_scheduled_tokens"),
        _dev(num_computed_tokens, torch.int32, "num_computed_tokens"),
        _dev(block_table, torch.int32, "block_table"), max(1, block_table.stride(0)), R,
        int(num_tokens),
        qsl_len, int(block_size), int(num_blocks),
        _dev(out["req_indices"], torch.int32), _dev(out["positions"], torch.int32),
        _dev(out["slot_mapping"], torch.int64), _dev(out["query_start_loc"], torch.int32),
        _dev(out["seq_lens"], torch.int32), _dev(out["logits_indices"], torch.int32),
        _stream(dev))
    _check(st, "pkv_prepare_inputs")
    return out


def prepare_inputs_and_plan(num_scheduled_tokens: torch.Tensor, num_computed_tokens: torch.Tensor,
                            block_table: torch.Tensor, *, num_tokens: int, block_size: int,
                            num_blocks: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            max_query_len: int, max_seq_len: int,
                            dtype: torch.dtype = torch.bfloat16, split_tokens: int = 0,
                            workspace: torch.Tensor | None = None, qsl_len: int | None = None,
                            out: dict | None = None) -> tuple[dict, torch.Tensor]:
    """pkv_prepare_inputs_and_plan: prepare_inputs and paged_attention_plan of
    one step in one launch.  Returns (the prepare outputs, the workspace that
    holds the work list); arguments as for the two calls."""
    R = int(num_scheduled_tokens.shape[0])
    dev = num_scheduled_tokens.device
    qsl_len = R + 1 if qsl_len is None else int(qsl_len)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {"req_indices": torch.empty(num_tokens, **i32),
               "positions": torch.empty(num_tokens, **i32),
               "slot_mapping": torch.empty(num_tokens, dtype=torch.int64, device=dev),
               "query_start_loc": torch.empty(qsl_len, **i32),
               "seq_lens": torch.empty(R, **i32),
               "logits_indices": torch.empty(R, **i32)}
    split_tokens = split_tokens_or_env(split_tokens)
    need = attention_workspace_bytes(R, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                     max_query_len, max_seq_len, split_tokens, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    assert block_table.dim() == 2 and (block_table.numel() == 0 or block_table.stride(1) == 1)
    st = load().pkv_prepare_inputs_and_plan(
        _dev(num_scheduled_tokens, torch.int32, "num_scheduled_tokens"),
        _dev(num_computed_tokens, torch.int32, "num_computed_tokens"),
        _dev(block_table, torch.int32, "block_table"), max(1, block_table.stride(0)), R,
        int(num_tokens), qsl_len, int(block_size), int(num_blocks),
        _dev(out["req_indices"], torch.int32), _dev(out["positions"], torch.int32),
        _dev(out["slot_mapping"], torch.int64), _dev(out["query_start_loc"], torch.int32),
        _dev(out["seq_lens"], torch.int32), _dev(out["logits_indices"], torch.int32),
        int(max_query_len), int(max_seq_len), int(num_q_heads), int(num_kv_heads),
        int(head_dim), _dtype_code(dtype), int(split_tokens), _dev(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "pkv_prepare_inputs_and_plan")
    return out, workspace


def prepare_input_ids(token_table: torch.Tensor, req_indices: torch.Tensor,
                      positions: torch.Tensor, seq_lens: torch.Tensor,
                      num_tokens_total: torch.Tensor, *, with_token_indices: bool = False,
                      out: dict | None = None) -> dict:
    """pkv_prepare_input_ids.  token_table: int32 [rows >= num_reqs, row_width]
    with contiguous rows; req_indices / positions / seq_lens as produced by
    prepare_inputs; num_tokens_total: int32 [num_reqs]."""
    T, R = int(req_indices.shape[0]), int(seq_lens.shape[0])
    assert token_table.dim() == 2 and token_table.shape[0] >= R
    assert token_table.numel() == 0 or token_table.is_contiguous()
    dev = req_indices.device
    if out is None:
        out = {"input_ids": torch.empty(T, dtype=torch.int32, device=dev),
               "discard_request_mask": torch.empty(R, dtype=torch.uint8, device=dev)}
        if with_token_indices:
            out["token_indices"] = torch.empty(T, dtype=torch.int64, device=dev)
    st = load().pkv_prepare_input_ids(
        _dev(token_table, torch.int32, "token_table"), int(token_table.shape[1]), R,
        _dev(req_indices, torch.int32, "req_indices"), _dev(positions, torch.int32, "positions"),
        T, _dev(seq_lens, torch.int32, "seq_lens"),
        _dev(num_tokens_total, torch.int32, "num_tokens_total"),
        _dev(out.get("token_indices"), torch.int64, "token_indices"),
        _dev(out["input_ids"], torch.int32, "input_ids"),
        _dev(out["discard_request_mask"], torch.uint8, "discard_request_mask"), _stream(dev))
    _check(st, "pkv_prepare_input_ids")
    return out


def paged_attention_plan(query_start_loc: torch.Tensor, seq_lens: torch.Tensor, *,
                         num_tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                         max_query_len: int, max_seq_len: int,
                         dtype: torch.dtype = torch.bfloat16, split_tokens: int = 0,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """pkv_paged_attention_plan: the batch's work list in ``workspace``
    (allocated when not given); pass it to paged_attention(..., planned=True,
    workspace=...) once per layer.  dtype is the q dtype (bf16 also for FP8
    pools)."""
    R = int(seq_lens.shape[0])
    split_tokens = split_tokens_or_env(split_tokens)
    need = attention_workspace_bytes(R, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                     max_query_len, max_seq_len, split_tokens, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=seq_lens.device)
    st = load().pkv_paged_attention_plan(
        _dev(query_start_loc, torch.int32, "query_start_loc"),
        _dev(seq_lens, torch.int32, "seq_lens"), R, int(num_tokens), int(max_query_len),
        int(max_seq_len), int(num_q_heads), int(num_kv_heads), int(head_dim), _dtype_code(dtype),
        int(split_tokens), _dev(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _stream(seq_lens.device))
    _check(st, "pkv_paged_attention_plan")
    return workspace


def _pool_block_size(key_cache: torch.Tensor, value_cache: torch.Tensor, head_dim: int) -> int:
    """Tokens per block of [nb, Hkv, head_dim * block_size] pools."""
    assert key_cache.dim() == 3 and value_cache.shape == key_cache.shape, \
        "pools are [num_blocks, num_kv_heads, head_dim * block_size]"
    assert key_cache.shape[2] % head_dim == 0
    return key_cache.shape[2] // head_dim


def _pool_block_bytes(key_cache: torch.Tensor, value_cache: torch.Tensor) -> int:
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    assert key_cache.shape[0] == value_cache.shape[0] and key_cache.dtype == value_cache.dtype
    nb = key_cache.shape[0]
    per = key_cache.numel() * key_cache.element_size() // max(1, nb)
    assert per == value_cache.numel() * value_cache.element_size() // max(1, nb)
    return per


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                block_pairs: torch.Tensor) -> None:
    """pkv_copy_blocks.  block_pairs: int32 [n, 2] (source, destination) on the
    pools' device; destinations distinct and never a source."""
    assert block_pairs.dim() == 2 and block_pairs.shape[1] == 2 and block_pairs.is_contiguous()
    st = load().pkv_copy_blocks(
        _dev(key_cache, name="key_cache"), _dev(value_cache, name="value_cache"),
        key_cache.shape[0], _pool_block_bytes(key_cache, value_cache),
        _dev(block_pairs, torch.int32, "block_pairs"), int(block_pairs.shape[0]),
        _stream(key_cache.device))
    _check(st, "pkv_copy_blocks")


def zero_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                block_ids: torch.Tensor) -> None:
    """pkv_zero_blocks.  block_ids: int32 [n] on the pools' device."""
    assert block_ids.dim() == 1 and block_ids.is_contiguous()
    st = load().pkv_zero_blocks(
        _dev(key_cache, name="key_cache"), _dev(value_cache, name="value_cache"),
        key_cache.shape[0], _pool_block_bytes(key_cache, value_cache),
        _dev(block_ids, torch.int32, "block_ids"), int(block_ids.shape[0]),
        _stream(key_cache.device))
    _check(st, "pkv_zero_blocks")


def kv_cache_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor, *,
                   block_size: int) -> None:
    """pkv_kv_cache_write.  key/value: [T, Hkv, d] with contiguous rows; pools
    [nb, Hkv, d * block_size] (workloads.key_pool / value_pool order)."""
    T, H, d = key.shape
    for t in (key, value):
        assert t.stride(2) == 1 and t.stride(1) == d, "heads and dims must be contiguous"
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    st = load().pkv_kv_cache_write(
        _dev(key, name="key"), _dev(value, name="value"), key.stride(0), value.stride(0),
        _dev(key_cache, key.dtype, "key_cache"), _dev(value_cache, key.dtype, "value_cache"),
        key_cache.shape[0], _dev(slot_mapping, torch.int64, "slot_mapping"), T, H, d,
        int(block_size), _dtype_code(key.dtype), _stream(key.device))
    _check(st, "pkv_kv_cache_write")


def kv_cache_write_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                       k_scale: torch.Tensor, v_scale: torch.Tensor, *, block_size: int) -> None:
    """pkv_kv_cache_write_fp8.  key/value: [T, Hkv, d] (bf16 or fp32) with
    contiguous rows; pools are uint8 tensors [nb, Hkv, d * 16] in the FP8
    layouts; scales are one-element float32 device tensors."""
    T, H, d = key.shape
    for t in (key, value):
        assert t.stride(2) == 1 and t.stride(1) == d, "heads and dims must be contiguous"
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    st = load().pkv_kv_cache_write_fp8(
        _dev(key, name="key"), _dev(value, name="value"), key.stride(0), value.stride(0),
        _dev(key_cache, torch.uint8, "key_cache"), _dev(value_cache, torch.uint8, "value_cache"),
        key_cache.shape[0], _dev(slot_mapping, torch.int64, "slot_mapping"), T, H, d,
        int(block_size), _dtype_code(key.dtype), _dev(k_scale, torch.float32, "k_scale"),
        _dev(v_scale, torch.float32, "v_scale"), _stream(key.device))
    _check(st, "pkv_kv_cache_write_fp8")


def split_tokens_or_env(split_tokens: int) -> int:
    """The context partition size a call uses: the argument, or when it is 0
    (the library's own choice) the PKV_SPLIT_TOKENS environment variable if set
    (a multiple of 32; for tuning without touching the caller)."""
    if split_tokens == 0:
        env = os.environ.get("PKV_SPLIT_TOKENS", "")
        if env:
            return int(env)
    return int(split_tokens)


def attention_workspace_bytes(num_reqs: int, num_tokens: int, num_q_heads: int,
                              num_kv_heads: int, head_dim: int, max_query_len: int,
                              max_seq_len: int, split_tokens: int = 0,
                              dtype: torch.dtype = torch.bfloat16) -> int:
    return int(load().pkv_paged_attention_workspace_bytes(
        num_reqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len, max_seq_len,
        split_tokens_or_env(split_tokens), _dtype_code(dtype)))


def paged_attention(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                    query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                    block_table: torch.Tensor, *, max_query_len: int, max_seq_len: int,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    split_tokens: int = 0, workspace: torch.Tensor | None = None,
                    k_scale: torch.Tensor | None = None,
                    v_scale: torch.Tensor | None = None, planned: bool = False) -> torch.Tensor:
    """pkv_paged_attention_varlen (or _fp8 when k_scale / v_scale are given).
    q: [T, Hq, d]; 16-bit pools: K [nb, Hkv, d * 16] in slabs of 32 dims
    (workloads.key_pool), V [nb, Hkv, d * 16] in tiles of 16 dims x 4 tokens
    (workloads.value_pool); FP8 pools (uint8): K and V [nb, Hkv, d * 16] in
    the FP8 layouts; scales: one-element float32 device tensors.
    planned=True: pkv_paged_attention_run over the work list a
    paged_attention_plan call left in ``workspace``."""
    T, Hq, d = q.shape
    nb, Hkv = key_cache.shape[0], key_cache.shape[1]
    bs = _pool_block_size(key_cache, value_cache, d)
    split_tokens = split_tokens_or_env(split_tokens)
    fp8 = k_scale is not None
    if fp8:
        assert v_scale is not None and key_cache.dtype == torch.uint8
    R = int(seq_lens.shape[0])
    assert q.stride(2) == 1 and q.stride(1) == d
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    assert block_table.dim() == 2 and block_table.stride(1) == 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    need = attention_workspace_bytes(R, T, Hq, Hkv, d, max_query_len, max_seq_len, split_tokens,
                                     q.dtype)
    if workspace is None and need:
        assert not planned, "a planned call runs over the plan's workspace"
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, name="workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args_head = (_dev(q, name="q"), q.stride(0),
                 _dev(key_cache, torch.uint8 if fp8 else q.dtype, "key_cache"),
                 _dev(value_cache, torch.uint8 if fp8 else q.dtype, "value_cache"), nb,
                 _dev(out, q.dtype, "out"), out.stride(0),
                 _dev(query_start_loc, torch.int32, "query_start_loc"),
                 _dev(seq_lens, torch.int32, "seq_lens"),
                 _dev(block_table, torch.int32, "block_table"), block_table.stride(0), R, T,
                 int(max_query_len), int(max_seq_len), Hq, Hkv, d, bs, float(scale))
    if planned:
        st = load().pkv_paged_attention_run(
            *args_head, BF16 if fp8 else _dtype_code(q.dtype),
            _dev(k_scale, torch.float32, "k_scale"), _dev(v_scale, torch.float32, "v_scale"),
            int(split_tokens), ws_ptr, ws_bytes, _stream(q.device))
        _check(st, "pkv_paged_attention_run")
        return out
    if fp8:
        st = load().pkv_paged_attention_varlen_fp8(
            *args_head, _dev(k_scale, torch.float32, "k_scale"),
            _dev(v_scale, torch.float32, "v_scale"), int(split_tokens), ws_ptr, ws_bytes,
            _stream(q.device))
        _check(st, "pkv_paged_attention_varlen_fp8")
        return out
    st = load().pkv_paged_attention_varlen(
        *args_head, _dtype_code(q.dtype), int(split_tokens), ws_ptr, ws_bytes, _stream(q.device))
    _check(st, "pkv_paged_attention_varlen")
    return out


def paged_attention_noalloc(q: torch.Tensor, key_cache: torch.Tensor,
                            value_cache: torch.Tensor, query_start_loc: torch.Tensor,
                            seq_lens: torch.Tensor, block_table: torch.Tensor, *,
                            out: torch.Tensor, max_query_len: int, max_seq_len: int,
                            scale: float | None = None, split_tokens: int = 0) -> torch.Tensor:
    """pkv_paged_attention_varlen_noalloc: paged_attention with the library's
    static scratch in place of a workspace.  ``out`` must be given (nothing
    is allocated on this path, here or in the library)."""
    T, Hq, d = q.shape
    nb, Hkv = key_cache.shape[0], key_cache.shape[1]
    bs = _pool_block_size(key_cache, value_cache, d)
    R = int(seq_lens.shape[0])
    assert q.stride(2) == 1 and q.stride(1) == d and out.shape == q.shape
    assert key_cache.is_contiguous() and value_cache.is_contiguous()
    assert block_table.dim() == 2 and block_table.stride(1) == 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = load().pkv_paged_attention_varlen_noalloc(
        _dev(q, name="q"), q.stride(0), _dev(key_cache, q.dtype, "key_cache"),
        _dev(value_cache, q.dtype, "value_cache"), nb, _dev(out, q.dtype, "out"), out.stride(0),
        _dev(query_start_loc, torch.int32, "query_start_loc"),
        _dev(seq_lens, torch.int32, "seq_lens"), _dev(block_table, torch.int32, "block_table"),
        block_table.stride(0), R, T, int(max_query_len), int(max_seq_len), Hq, Hkv, d, bs,
        float(scale), _dtype_code(q.dtype), int(split_tokens_or_env(split_tokens)),
        _stream(q.device))
    _check(st, "pkv_paged_attention_varlen_noalloc")
    return out
