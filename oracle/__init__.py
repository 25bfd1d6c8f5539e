"""fp64 CPU oracle for the paged KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
the two share no code: this wrapper talks to ``liboracle.so`` (built from
``oracle.c`` with gcc) and to nothing else.

What each function computes, and where on the pages it comes from, is stated
in ``oracle.c``:

* :func:`prepare`   -- flat-batch index tensors ("Building the Batch", "How
  they are computed"; "vLLM's Model Runner -- the Persistent Batch, in
  Source", "The two things this method returns").
* :func:`kv_write`  -- token-granular scatter into the block pool ("Inside
  vLLM: Following One Request from the API to GPU Execution", Part 5).
* :func:`attention` -- gather each request's blocks, then naive causal
  softmax attention in fp64 ("How vLLM Works Internally: A Deep Dive", "How
  the Kernel Works").

Every function is pinned by ``tests/test_oracle_pins.py`` to values the pages
print, to closed forms, to torch's own fp64 attention and to invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants mistakes in copies of oracle.c points this at the mutant build.
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or _DEFAULT_LIB

OK = 0
ERR_ARG = 1
ERR_RANGE = 2
ERR_DUP = 3
ERR_PRECOND = 4
ERR_NOMEM = 5

F32 = 0
BF16 = 1
FP8 = 2


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        names = {ERR_ARG: "invalid argument", ERR_RANGE: "index out of range",
                 ERR_DUP: "duplicate slot", ERR_PRECOND: "precondition violated",
                 ERR_NOMEM: "out of memory"}
        super().__init__(f"oracle {what}: {names.get(code, code)}")
        self.code = code


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, OpenMP).  Always rebuilds."""
    tmp = _DEFAULT_LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_prepare.argtypes = [P, P, P, i64, i32, i32, i32, i32, i64, P, P, P, P, P, P, P]
    lib.orc_prepare.restype = ctypes.c_int
    lib.orc_kv_write.argtypes = [P, P, i64, i64, P, P, i64, P, i32, i32, i32, i32, i32]
    lib.orc_kv_write.restype = ctypes.c_int
    lib.orc_attention.argtypes = [P, i64, P, P, i32, P, P, P, i64, i32, i32, i32, i32, i32,
                                  i32, i64, f64, P, i32, P, i32]
    lib.orc_attention.restype = ctypes.c_int
    lib.orc_attention_kv.argtypes = [P, i64, P, P, i32, i32, f64, f64, P, P, P, i64, i32, i32,
                                     i32, i32, i32, i32, i64, f64, P, i32, P, i32]
    lib.orc_attention_kv.restype = ctypes.c_int
    lib.orc_kv_write_fp8.argtypes = [P, P, i64, i64, P, P, i64, P, i32, i32, i32, i32, i32,
                                     ctypes.c_float, ctypes.c_float]
    lib.orc_kv_write_fp8.restype = ctypes.c_int
    lib.orc_fp8_decode.argtypes = [ctypes.c_uint8]
    lib.orc_fp8_decode.restype = f64
    lib.orc_fp8_encode.argtypes = [ctypes.c_float]
    lib.orc_fp8_encode.restype = ctypes.c_uint8
    lib.orc_input_ids.argtypes = [P, i64, i32, P, P, i32, P, P, P, P, P]
    lib.orc_input_ids.restype = ctypes.c_int
    lib.orc_copy_blocks.argtypes = [P, P, i64, i64, P, i32]
    lib.orc_copy_blocks.restype = ctypes.c_int
    lib.orc_zero_blocks.argtypes = [P, P, i64, i64, P, i32]
    lib.orc_zero_blocks.restype = ctypes.c_int
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _ptr(a) -> int | None:
    """Address of a contiguous numpy array or CPU torch tensor."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
        return a.ctypes.data
    # torch tensor (CPU)
    assert a.device.type == "cpu" and a.is_contiguous(), "oracle needs contiguous CPU tensors"
    return a.data_ptr()


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def prepare(num_scheduled_tokens, num_computed_tokens, block_table, block_size: int,
            num_blocks: int, qsl_len: int | None = None) -> dict:
    """Flat-batch index tensors for one step; see ``orc_prepare`` in oracle.c."""
    nst = _i32(num_scheduled_tokens)
    nct = _i32(num_computed_tokens)
    R = int(nst.shape[0])
    bt = _i32(block_table).reshape(R, -1) if R else np.zeros((0, 1), np.int32)
    T = int(nst.sum())
    qsl_len = R + 1 if qsl_len is None else int(qsl_len)
    out = {
        "req_indices": np.zeros(T, np.int32),
        "positions": np.zeros(T, np.int32),
        "slot_mapping": np.zeros(T, np.int64),
        "query_start_loc": np.zeros(qsl_len, np.int32),
        "seq_lens": np.zeros(R, np.int32),
        "logits_indices": np.zeros(R, np.int32),
    }
    n_out = ctypes.c_int64(0)
    rc = _load().orc_prepare(
        _ptr(nst), _ptr(nct), _ptr(bt), bt.shape[1], bt.shape[1], R, qsl_len, block_size,
        num_blocks, _ptr(out["req_indices"]), _ptr(out["positions"]), _ptr(out["slot_mapping"]),
        _ptr(out["query_start_loc"]), _ptr(out["seq_lens"]), _ptr(out["logits_indices"]),
        ctypes.addressof(n_out))
    if rc != OK:
        raise OracleError(rc, "prepare")
    assert n_out.value == T
    return out


def input_ids(token_table, req_indices, positions, seq_lens, num_tokens_total) -> dict:
    """Token ids of the flat rows and the discard mask; see ``orc_input_ids``.
    ``token_table`` is int32 [R, row_width] (request r in row r)."""
    table = _i32(token_table)
    R = int(np.asarray(seq_lens).shape[0])
    table = table.reshape(max(R, 1) if table.size else 0, -1) if table.ndim == 1 else table
    ri, pos = _i32(req_indices), _i32(positions)
    T = int(ri.shape[0])
    out = {"token_indices": np.zeros(T, np.int64), "input_ids": np.zeros(T, np.int32),
           "discard_request_mask": np.zeros(R, np.uint8)}
    rc = _load().orc_input_ids(_ptr(table), table.shape[1], R, _ptr(ri), _ptr(pos), T,
                               _ptr(_i32(seq_lens)), _ptr(_i32(num_tokens_total)),
                               _ptr(out["token_indices"]), _ptr(out["input_ids"]),
                               _ptr(out["discard_request_mask"]))
    if rc != OK:
        raise OracleError(rc, "input_ids")
    return out


def _block_bytes(pool) -> int:
    import torch
    if isinstance(pool, np.ndarray):
        return pool[0].nbytes if pool.shape[0] else 1
    return pool[0].numel() * pool.element_size() if pool.shape[0] else 1


def copy_blocks(key_cache, value_cache, pairs) -> None:
    """Whole-block copies src -> dst in both pools, in order; see ``orc_copy_blocks``."""
    pr = _i32(pairs).reshape(-1, 2)
    rc = _load().orc_copy_blocks(_ptr(key_cache), _ptr(value_cache), key_cache.shape[0],
                                 _block_bytes(key_cache), _ptr(pr), pr.shape[0])
    if rc != OK:
        raise OracleError(rc, "copy_blocks")


def zero_blocks(key_cache, value_cache, block_ids) -> None:
    """Clear the listed blocks of both pools; see ``orc_zero_blocks``."""
    ids = _i32(block_ids).reshape(-1)
    rc = _load().orc_zero_blocks(_ptr(key_cache), _ptr(value_cache), key_cache.shape[0],
                                 _block_bytes(key_cache), _ptr(ids), ids.shape[0])
    if rc != OK:
        raise OracleError(rc, "zero_blocks")


def kv_write(key, value, key_cache, value_cache, slot_mapping, block_size: int) -> None:
    """Scatter new K/V rows into the caches in place; see ``orc_kv_write``.

    ``key``/``value`` are [T, Hkv, d] CPU tensors or arrays (any 2- or 4-byte
    dtype; bytes are copied unchanged).  Both caches hold nb * Hkv runs of
    d * bs elements ([nb, Hkv, d * bs]): a K run in slabs of 32 dims
    ([d / 32][bs][32], plain [bs][d] when 32 does not divide d), a V run in
    tiles of 16 dims x 4 tokens ([d / 16][bs / 4][16][4], plain [d][bs] when
    16 does not divide d or 4 does not divide bs).
    """
    T, H, d = key.shape
    nb = key_cache.shape[0]
    slots = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    esz = key.element_size() if hasattr(key, "element_size") else key.itemsize
    rc = _load().orc_kv_write(_ptr(key), _ptr(value), H * d, H * d, _ptr(key_cache),
                              _ptr(value_cache), nb, _ptr(slots), T, H, d, block_size, esz)
    if rc != OK:
        raise OracleError(rc, "kv_write")


def fp8_decode(code: int) -> float:
    """Value of one FP8 E4M3 code; see ``orc_fp8_decode``."""
    return float(_load().orc_fp8_decode(int(code)))


def fp8_encode(x: float) -> int:
    """E4M3 code of a binary32 value (nearest, ties to even, saturating); see
    ``orc_fp8_encode``."""
    return int(_load().orc_fp8_encode(float(np.float32(x))))


def kv_write_fp8(key, value, key_cache, value_cache, slot_mapping, block_size: int,
                 k_scale: float, v_scale: float) -> None:
    """FP8 form of :func:`kv_write`; see ``orc_kv_write_fp8``.

    ``key``/``value`` are [T, Hkv, d] bf16 or fp32; the pools are uint8 arrays or
    tensors of [nb, Hkv, d * bs] bytes in the FP8 layouts (K runs
    [d / 64][bs][64], V runs as in ``orc_v8_byte``); the scales are binary32
    values.
    """
    T, H, d = key.shape
    nb = key_cache.shape[0]
    slots = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    esz = key.element_size() if hasattr(key, "element_size") else key.itemsize
    rc = _load().orc_kv_write_fp8(_ptr(key), _ptr(value), H * d, H * d, _ptr(key_cache),
                                  _ptr(value_cache), nb, _ptr(slots), T, H, d, block_size, esz,
                                  float(np.float32(k_scale)), float(np.float32(v_scale)))
    if rc != OK:
        raise OracleError(rc, "kv_write_fp8")


def attention(q, key_cache, value_cache, query_start_loc, seq_lens, block_table,
              block_size: int, scale: float, rows=None, num_threads: int = 0,
              kv_scales=None) -> np.ndarray:
    """fp64 causal paged attention; see ``orc_attention`` / ``orc_attention_kv``.

    ``q`` is [T, Hq, d] (fp32 or bf16 CPU tensor, or float32 numpy array).
    With ``kv_scales = (k_scale, v_scale)`` the pools hold FP8 E4M3 bytes
    (uint8) in the FP8 layouts and every element reads as code value x scale.
    Returns a float64 array [len(rows), Hq, d] (all T rows when ``rows`` is None).
    """
    T, Hq, d = q.shape
    nb, Hkv = key_cache.shape[0], key_cache.shape[1]
    if isinstance(q, np.ndarray):
        assert q.dtype == np.float32
        dtype = F32
    else:
        import torch
        dtype = {torch.float32: F32, torch.bfloat16: BF16}[q.dtype]
        if kv_scales is None:
            assert key_cache.dtype == q.dtype and value_cache.dtype == q.dtype
    kv_dtype, ks, vs = dtype, 1.0, 1.0
    if kv_scales is not None:
        kv_dtype = FP8
        ks, vs = (float(np.float32(x)) for x in kv_scales)
    qsl = _i32(query_start_loc)
    sl = _i32(seq_lens)
    R = int(sl.shape[0])
    bt = _i32(block_table).reshape(R, -1)
    if rows is None:
        sel = None
        n = int(qsl[R])
    else:
        sel = _i32(rows)
        n = int(sel.shape[0])
    out = np.zeros((n, Hq, d), np.float64)
    rc = _load().orc_attention_kv(
        _ptr(q), Hq * d, _ptr(key_cache), _ptr(value_cache), dtype, kv_dtype, ks, vs, _ptr(qsl),
        _ptr(sl), _ptr(bt), bt.shape[1], bt.shape[1], R, Hq, Hkv, d, block_size, nb,
        float(scale), _ptr(sel), n, _ptr(out), int(num_threads))
    if rc != OK:
        raise OracleError(rc, "attention")
    return out
