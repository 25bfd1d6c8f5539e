"""Seeded synthetic inputs for the paged KV-cache hot path.

This module builds inputs only: request lengths, block tables, a pre-filled
block pool, and the new Q/K/V rows of one step.  It holds none of the
method's arithmetic (no positions, no slot mapping, no attention) and is the
one piece of code that both the HIP library's tests and the fp64 oracle's
tests use.

Recipe (every configuration):

* integer structure from ``numpy.random.default_rng(seed)``, drawn in the order
  lengths -> block permutation;
* bulk values from a ``torch.Generator`` seeded with ``seed`` on the target
  device, drawn in the order cache fill -> Q -> K_new -> V_new, as fp32
  N(0, 1) samples rounded to the working dtype (round-to-nearest-even for
  bf16);
* a request's physical blocks are dealt from a random permutation of the pool,
  in request order; table columns a request does not use hold -1;
* pool slots that hold no history (positions >= num_computed_tokens of the
  owning request, whole blocks no request owns, and the slack blocks) are
  poisoned with NaN, so a kernel that reads outside a request's context, or
  lets a masked value into a sum, produces NaN.

Layouts (the library's interface, not part of the method): new rows are
[T, H, d]; the pools are [num_blocks, Hkv, d * block_size], the K pool in
slabs of 32 dims per (block, head) run (``key_pool``), the V pool in tiles of
16 dims x 4 tokens (``value_pool``).

FP8 pools (``to_fp8``): the same history as E4M3 codes of value / scale,
converted by torch's float8_e4m3fn (after clamping to +-448; NaN poison stays
NaN), as uint8 tensors [num_blocks, Hkv, d * 16]: K in slabs of 64 dims (per
run: dim / 64, token, dim % 64), V in the documented FP8 V order (per run:
dim / 64, token / 4, dim % 16, (dim / 16) % 4, token % 4).

The five named configurations are the shapes of the pages' workloads: a
three-request step of the worked example ("Building the Batch", "How they are
computed"), 13B- and 8B-shaped decode batches, one 5,000-token prompt chunk
next to 200 decodes ("Building the Batch", "Why flatten"), and long contexts
with shared prefix blocks ("How vLLM Works Internally: A Deep Dive",
"Copy-on-Write for Beam Search").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16


@dataclass
class Workload:
    name: str
    num_scheduled_tokens: np.ndarray   # int32 [R]
    num_computed_tokens: np.ndarray    # int32 [R]
    block_table: np.ndarray            # int32 [R, max_blocks], unused entries -1
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: torch.dtype
    scale: float
    seed: int
    q: torch.Tensor = None             # [T, Hq, d]
    key: torch.Tensor = None           # [T, Hkv, d]
    value: torch.Tensor = None         # [T, Hkv, d]
    key_cache: torch.Tensor = None     # [nb, Hkv, d * bs] (key_pool order), or FP8 codes
    value_cache: torch.Tensor = None   # [nb, Hkv, d * bs] (value_pool order), or FP8 codes
    notes: dict = field(default_factory=dict)
    kv_scales: tuple = None            # (k_scale, v_scale) when the pools hold FP8 codes

    @property
    def num_reqs(self) -> int:
        return int(self.num_scheduled_tokens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.num_scheduled_tokens.sum())

    @property
    def max_query_len(self) -> int:
        return int(self.num_scheduled_tokens.max()) if self.num_reqs else 0

    @property
    def max_seq_len(self) -> int:
        if not self.num_reqs:
            return 0
        return int((self.num_scheduled_tokens + self.num_computed_tokens).max())

    def to(self, device) -> "Workload":
        for name in ("q", "key", "value", "key_cache", "value_cache"):
            setattr(self, name, getattr(self, name).to(device))
        return self


def _blocks_for(length: int, bs: int) -> int:
    return (length + bs - 1) // bs


def _randn(gen: torch.Generator, shape, dtype, device) -> torch.Tensor:
    """fp32 N(0,1) rounded to ``dtype``, drawn in chunks to bound fp32 temporaries."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for start in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, dtype=torch.float32,
                                            device=device).to(dtype)
    return out


def build(name: str, nst, nct, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
          dtype=torch.bfloat16, seed: int = 0, block_size: int = BLOCK_SIZE,
          pool_slack: float = 1.0, shared_prefix_groups=None, device="cpu",
          scale: float | None = None, extra_table_cols: int = 0,
          rng: np.random.Generator | None = None) -> Workload:
    """Build one seeded step.

    ``shared_prefix_groups``: optional list of (request ids, prefix tokens); the
    listed requests use the same physical blocks for their first ``prefix``
    tokens (a whole number of blocks), as requests with a common prompt prefix
    do after prefix caching.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    nst = np.asarray(nst, dtype=np.int32)
    nct = np.asarray(nct, dtype=np.int32)
    R = int(nst.shape[0])
    bs = block_size
    seq = (nst.astype(np.int64) + nct)
    need = [_blocks_for(int(L), bs) for L in seq]

    # Which logical blocks come from a shared run: owner of each shared group first.
    shared_of = {}
    n_shared_blocks = 0
    for members, prefix in (shared_prefix_groups or []):
        assert prefix % bs == 0
        nblk = prefix // bs
        for m in members:
            assert nct[m] >= prefix, "new tokens must not land in shared blocks"
            shared_of[m] = (members[0], nblk)
        n_shared_blocks += nblk
    unique_need = sum(need[r] - (shared_of[r][1] if r in shared_of else 0) for r in range(R))
    total_need = unique_need + n_shared_blocks
    num_blocks = max(1, int(math.ceil(total_need * pool_slack)))

    perm = rng.permutation(num_blocks).astype(np.int32)
    cols = max(need) + extra_table_cols if R else 1
    table = np.full((R, max(cols, 1)), -1, dtype=np.int32)
    cursor = 0
    shared_runs = {}
    for r in range(R):
        start_col = 0
        if r in shared_of:
            owner, nblk = shared_of[r]
            if owner not in shared_runs:
                shared_runs[owner] = perm[cursor:cursor + nblk].copy()
                cursor += nblk
            table[r, :nblk] = shared_runs[owner]
            start_col = nblk
        k = need[r] - start_col
        table[r, start_col:need[r]] = perm[cursor:cursor + k]
        cursor += k
    assert cursor == total_need

    # History mask: slot (block, offset) holds a value iff it is at a position
    # below num_computed_tokens of a request that owns the block.
    history = np.zeros((num_blocks, bs), dtype=bool)
    for r in range(R):
        full = int(nct[r]) // bs
        rem = int(nct[r]) % bs
        if full:
            history[table[r, :full]] = True
        if rem:
            history[table[r, full], :rem] = True

    H, Hkv, d = num_q_heads, num_kv_heads, head_dim
    T = int(nst.sum())
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    kc = _randn(gen, (num_blocks, Hkv, bs, d), dtype, device)
    vc = _randn(gen, (num_blocks, Hkv, d, bs), dtype, device)
    hist = torch.from_numpy(history).to(device)
    kc.masked_fill_(~hist[:, None, :, None], float("nan"))
    vc.masked_fill_(~hist[:, None, None, :], float("nan"))
    kc = key_pool(kc)
    vc = value_pool(vc)
    q = _randn(gen, (T, H, d), dtype, device)
    k_new = _randn(gen, (T, Hkv, d), dtype, device)
    v_new = _randn(gen, (T, Hkv, d), dtype, device)

    wl = Workload(name=name, num_scheduled_tokens=nst, num_computed_tokens=nct,
                  block_table=table, num_blocks=num_blocks, num_q_heads=H,
                  num_kv_heads=Hkv, head_dim=d, block_size=bs, dtype=dtype,
                  scale=(1.0 / math.sqrt(d)) if scale is None else scale, seed=seed,
                  q=q, key=k_new, value=v_new, key_cache=kc, value_cache=vc)
    wl.notes["shared_blocks"] = n_shared_blocks
    wl.notes["unique_blocks"] = unique_need
    return wl


def _key_slab(head_dim: int) -> int:
    return 32 if head_dim % 32 == 0 else head_dim


def key_pool(logical: torch.Tensor) -> torch.Tensor:
    """A 16-bit or fp32 K pool from its logical form [nb, Hkv, bs, d] (element
    [b, h, tok, dim]): [nb, Hkv, d * bs], each (block, head) run in slabs of
    32 dims, [dim / 32][tok][dim % 32] (plain [tok][dim] when 32 does not
    divide d)."""
    nb, H, bs, d = logical.shape
    kw = _key_slab(d)
    x = logical.reshape(nb, H, bs, d // kw, kw).transpose(2, 3)
    return x.reshape(nb, H, d * bs).contiguous()


def key_logical(pool: torch.Tensor, head_dim: int, block_size: int) -> torch.Tensor:
    """The inverse of key_pool: [nb, Hkv, bs, d] from a K pool."""
    nb, H = pool.shape[0], pool.shape[1]
    kw = _key_slab(head_dim)
    x = pool.reshape(nb, H, head_dim // kw, block_size, kw).transpose(2, 3)
    return x.reshape(nb, H, block_size, head_dim).contiguous()


def fp8_key_pool(logical: torch.Tensor) -> torch.Tensor:
    """An FP8 K pool from logical codes [nb, Hkv, 16, d] (d a multiple of 64):
    [nb, Hkv, d * 16], each run in slabs of 64 dims, [dim / 64][tok][dim % 64]."""
    nb, H, bs, d = logical.shape
    assert bs == 16 and d % 64 == 0
    x = logical.reshape(nb, H, bs, d // 64, 64).transpose(2, 3)
    return x.reshape(nb, H, d * bs).contiguous()


def _value_tiles(head_dim: int, block_size: int) -> tuple[int, int]:
    return (16 if head_dim % 16 == 0 else head_dim), (4 if block_size % 4 == 0 else block_size)


def value_pool(logical: torch.Tensor) -> torch.Tensor:
    """A 16-bit or fp32 V pool from its logical form [nb, Hkv, d, bs] (element
    [b, h, dim, tok]): [nb, Hkv, d * bs], each (block, head) run in tiles of
    16 dims x 4 tokens, [dim / 16][tok / 4][dim % 16][tok % 4] (one tile
    spans all dims when 16 does not divide d, all tokens when 4 does not
    divide bs)."""
    nb, H, d, bs = logical.shape
    dw, tg = _value_tiles(d, bs)
    x = logical.reshape(nb, H, d // dw, dw, bs // tg, tg).transpose(3, 4)
    return x.reshape(nb, H, d * bs).contiguous()


def value_logical(pool: torch.Tensor, head_dim: int, block_size: int) -> torch.Tensor:
    """The inverse of value_pool: [nb, Hkv, d, bs] from a V pool."""
    nb, H = pool.shape[0], pool.shape[1]
    dw, tg = _value_tiles(head_dim, block_size)
    x = pool.reshape(nb, H, head_dim // dw, block_size // tg, dw, tg).transpose(3, 4)
    return x.reshape(nb, H, head_dim, block_size).contiguous()


def fp8_value_order(head_dim: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """For each byte of an FP8 V run, the flat index dim * block_size + token of
    the element it holds (the documented FP8 V order)."""
    assert block_size == 16 and head_dim % 64 == 0
    order = np.empty(head_dim * block_size, np.int64)
    for dim in range(head_dim):
        for tok in range(block_size):
            byte = ((((dim // 64) * 4 + tok // 4) * 16 + dim % 16) * 4 + (dim // 16) % 4) * 4 \
                + tok % 4
            order[byte] = dim * block_size + tok
    return order


def to_fp8(wl: Workload, k_scale: float, v_scale: float) -> Workload:
    """The same step with FP8 pools: every history element as the E4M3 code of
    value / scale (torch's float8_e4m3fn conversion).  New rows stay bf16."""
    assert wl.dtype == torch.bfloat16
    nb, H = wl.key_cache.shape[0], wl.key_cache.shape[1]
    bs, d = wl.block_size, wl.head_dim

    def codes(x, scale):
        return (x.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    kc = fp8_key_pool(codes(key_logical(wl.key_cache, d, bs), k_scale))
    order = torch.from_numpy(fp8_value_order(d, bs)).to(wl.value_cache.device)
    logical_v = value_logical(wl.value_cache, d, bs)
    vc = codes(logical_v, v_scale).reshape(nb, H, d * bs)[:, :, order].contiguous()
    out = Workload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__})
    out.name = wl.name + "-fp8"
    out.key_cache, out.value_cache = kc, vc
    out.kv_scales = (float(np.float32(k_scale)), float(np.float32(v_scale)))
    out.notes = dict(wl.notes)
    return out


def select(wl: Workload, reqs, name: str | None = None) -> Workload:
    """The sub-batch of requests ``reqs`` (in order) over the same block pools:
    their scheduled rows of Q/K/V, counts and block-table rows."""
    reqs = np.asarray(reqs, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(wl.num_scheduled_tokens)]).astype(np.int64)
    rows = np.concatenate([np.arange(starts[r], starts[r + 1]) for r in reqs]) if len(reqs) \
        else np.zeros(0, np.int64)
    idx = torch.from_numpy(rows).to(wl.q.device)
    sub = Workload(name=name or f"{wl.name}[{len(reqs)} requests]",
                   num_scheduled_tokens=wl.num_scheduled_tokens[reqs].copy(),
                   num_computed_tokens=wl.num_computed_tokens[reqs].copy(),
                   block_table=np.ascontiguousarray(wl.block_table[reqs]),
                   num_blocks=wl.num_blocks, num_q_heads=wl.num_q_heads,
                   num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
                   block_size=wl.block_size, dtype=wl.dtype, scale=wl.scale, seed=wl.seed,
                   q=wl.q[idx].contiguous(), key=wl.key[idx].contiguous(),
                   value=wl.value[idx].contiguous(), key_cache=wl.key_cache,
                   value_cache=wl.value_cache, notes=dict(wl.notes), kv_scales=wl.kv_scales)
    return sub


# ---------------------------------------------------------------------------
# The five named configurations
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "worked-example step: nst [2,5,3], nct [14,0,9], Hq 4 / Hkv 2, d 64, fp32",
    2: "decode batch: 64 x 1 token, context U[512,2048], Hq 40 / Hkv 40, d 128, bf16",
    3: "GQA decode batch: 256 x 1 token, context 4096, Hq 32 / Hkv 8, d 128, bf16",
    4: "mixed step: 5000-token chunk at 3000 computed + 200 decodes U[1024,8192], "
       "Hq 32 / Hkv 8, d 128, bf16",
    5: "long context + shared prefix: 16 decodes at 32768 in 4 groups sharing 16384 "
       "tokens + a 2048-token prefill, Hq 64 / Hkv 8, d 128, bf16",
}


def config(idx: int, device="cpu", seed: int | None = None) -> Workload:
    """Configuration ``idx`` (1..5) with seed 1000 + idx unless given."""
    seed = 1000 + idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if idx == 1:
        return build("cfg1", [2, 5, 3], [14, 0, 9], num_q_heads=4, num_kv_heads=2,
                     head_dim=64, dtype=torch.float32, seed=seed, device=device,
                     pool_slack=16 / 3, rng=rng)
    if idx == 2:
        ctx = rng.integers(512, 2048, size=64, endpoint=True)
        return build("cfg2", np.ones(64, np.int32), (ctx - 1).astype(np.int32),
                     num_q_heads=40, num_kv_heads=40, head_dim=128, seed=seed,
                     device=device, pool_slack=1.25, rng=rng)
    if idx == 3:
        return build("cfg3", np.ones(256, np.int32), np.full(256, 4095, np.int32),
                     num_q_heads=32, num_kv_heads=8, head_dim=128, seed=seed,
                     device=device, rng=rng)
    if idx == 4:
        ctx = rng.integers(1024, 8192, size=200, endpoint=True)
        nst = np.concatenate([[5000], np.ones(200, np.int64)]).astype(np.int32)
        nct = np.concatenate([[3000], ctx - 1]).astype(np.int32)
        return build("cfg4", nst, nct, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     seed=seed, device=device, pool_slack=1.25, rng=rng)
    if idx == 5:
        nst = np.concatenate([np.ones(16, np.int64), [2048]]).astype(np.int32)
        nct = np.concatenate([np.full(16, 32767), [0]]).astype(np.int32)
        groups = [(list(range(4 * g, 4 * g + 4)), 16384) for g in range(4)]
        return build("cfg5", nst, nct, num_q_heads=64, num_kv_heads=8, head_dim=128,
                     seed=seed, device=device, shared_prefix_groups=groups, rng=rng)
    raise ValueError(f"no configuration {idx}")


def config_structure(idx: int, seed: int | None = None) -> dict:
    """Host-side integer structure of configuration ``idx`` without any bulk tensors
    (request lengths and the block-table shape), for sizing and byte counts."""
    seed = 1000 + idx if seed is None else seed
    rng = np.random.default_rng(seed)
    if idx == 1:
        nst, nct = np.array([2, 5, 3]), np.array([14, 0, 9])
    elif idx == 2:
        ctx = rng.integers(512, 2048, size=64, endpoint=True)
        nst, nct = np.ones(64, np.int64), ctx - 1
    elif idx == 3:
        nst, nct = np.ones(256, np.int64), np.full(256, 4095)
    elif idx == 4:
        ctx = rng.integers(1024, 8192, size=200, endpoint=True)
        nst = np.concatenate([[5000], np.ones(200, np.int64)])
        nct = np.concatenate([[3000], ctx - 1])
    elif idx == 5:
        nst = np.concatenate([np.ones(16, np.int64), [2048]])
        nct = np.concatenate([np.full(16, 32767), [0]])
    else:
        raise ValueError(idx)
    heads = {1: (4, 2, 64), 2: (40, 40, 128), 3: (32, 8, 128), 4: (32, 8, 128),
             5: (64, 8, 128)}[idx]
    return {"num_scheduled_tokens": nst.astype(np.int32),
            "num_computed_tokens": nct.astype(np.int32),
            "num_q_heads": heads[0], "num_kv_heads": heads[1], "head_dim": heads[2],
            "dtype": torch.float32 if idx == 1 else torch.bfloat16}
