"""Seeded synthetic workloads for attention over a paged KV cache.

Every workload is a batch of requests in the packed varlen form the vLLM pages
describe ("vllm v1 源码精读（三）", §3.4 and §4.2; "Inside vLLM", §3.4):

* ``pool``           [num_blocks, 2, block_size, num_kv_heads, head_dim] KV cache
                     (index 0 = K, 1 = V), storage dtype bits;
* ``block_table``    int32 [R, W], row r maps logical block j to a physical
                     block id, unused entries are -1;
* ``seq_lens``       int32 [R], keys the request's last query can see,
                     including the tokens written this step;
* ``num_computed``   int32 [R], tokens already in the cache before this step;
* ``query_start_loc``int32 [R+1], prefix of the per-request query counts;
* ``q``              [T, Hq, D] queries of this step (varlen packed);
* ``k_new, v_new``   [T, Hkv, D] keys/values of this step's tokens.

The generator only draws numbers and allocates blocks: values are N(0, 1)
rounded to the storage dtype, lengths are uniform integers, physical block ids
come from a seeded permutation of the pool (so tables are scattered and
distinct).  Blocks no request owns are filled with NaN so that any stray read
shows up in the result.  Nothing here computes slots, scatters or attends.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

_NAN_BITS = {"bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00)}


def storage_dtype(dtype: str):
    """numpy dtype holding one element of a cache/query of ``dtype``."""
    if dtype == "f32":
        return np.float32
    if dtype in ("bf16", "f16"):
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def element_size(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns.  Inputs here are finite normals, so no NaN
    handling is needed beyond keeping NaN inputs NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = _NAN_BITS["bf16"]
    return out


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (numpy rounds to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    return f16_bits_from_f32(x)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


_FILL_CHUNK = 1024  # blocks per independently seeded chunk of pool values


def _fill_blocks(pool: np.ndarray, ids: np.ndarray, seed: int, dtype: str) -> None:
    """pool[ids] = N(0,1) values.  Chunk i of ``_FILL_CHUNK`` ids draws from its
    own stream seeded by (seed, i), so the result does not depend on how many
    threads fill the chunks."""
    blk_shape = pool.shape[1:]
    starts = list(range(0, ids.size, _FILL_CHUNK))

    def work(i):
        sub = ids[starts[i]:starts[i] + _FILL_CHUNK]
        rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED, i]))
        pool[sub] = _normal(rng, (sub.size,) + blk_shape, dtype)

    threads = min(16, os.cpu_count() or 1, max(1, len(starts)))
    if threads <= 1:
        for i in range(len(starts)):
            work(i)
    else:
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(len(starts))))


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens: np.ndarray
    num_computed: np.ndarray
    query_start_loc: np.ndarray
    block_table: np.ndarray
    pool: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    seed: int
    meta: Dict = dataclasses.field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int32)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def is_decode_only(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    @property
    def used_blocks(self) -> np.ndarray:
        """Distinct physical blocks referenced by the tables (ids >= 0)."""
        bt = self.block_table
        return np.unique(bt[bt >= 0])


# --------------------------------------------------------------------------
# generic builder
# --------------------------------------------------------------------------


def build_workload(
    name: str,
    *,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    num_blocks: int,
    requests: Sequence[Tuple[int, int]],
    seed: int,
    block_size: int = 16,
    table_width: Optional[int] = None,
    shared_prefix_blocks: int = 0,
    scale: Optional[float] = None,
    fill_unused: str = "nan",
    meta: Optional[Dict] = None,
    values: bool = True,
) -> Workload:
    """Build a batch from ``requests`` = [(num_computed, q_len), ...].

    Each request owns ceil(seq_len / block_size) blocks (the allocation rule
    of "Inside vLLM" §3.3).  With ``shared_prefix_blocks`` = S, the first S
    logical blocks of every request are the same S physical blocks (a shared
    system prompt, as with prefix caching); the rest are private.
    Physical ids are drawn without replacement from a seeded permutation of
    the pool: shared ids first, then each request's private ids in order.
    With ``values=False`` only the metadata is built (pool, q, k_new, v_new
    are None); the metadata is the same as with values.
    """
    rng = np.random.default_rng(seed)
    R = len(requests)
    num_computed = np.array([c for c, _ in requests], dtype=np.int32).reshape(R)
    q_lens = np.array([n for _, n in requests], dtype=np.int32).reshape(R)
    seq_lens = (num_computed + q_lens).astype(np.int32)
    qsl = np.zeros(R + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)

    nblk = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    width = table_width if table_width is not None else max([1] + nblk)
    if max([0] + nblk) > width:
        raise ValueError(f"{name}: table width {width} < {max(nblk)} blocks")
    S = shared_prefix_blocks
    if S and any(n < S for n in nblk):
        raise ValueError(f"{name}: a request is shorter than the shared prefix")
    need = S + sum(n - S for n in nblk)
    if need > num_blocks:
        raise ValueError(f"{name}: needs {need} blocks, pool has {num_blocks}")

    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((R, width), -1, dtype=np.int32)
    shared = perm[:S]
    nxt = S
    for r in range(R):
        table[r, :S] = shared
        own = nblk[r] - S
        table[r, S:nblk[r]] = perm[nxt:nxt + own]
        nxt += own

    meta = dict(meta or {})
    meta["blocks_used"] = int(need)
    meta["shared_prefix_blocks"] = int(S)
    if not values:
        return Workload(
            name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
            head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
            scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
            seq_lens=seq_lens, num_computed=num_computed, query_start_loc=qsl,
            block_table=table, pool=None, q=None, k_new=None, v_new=None, seed=seed,
            meta=meta)

    # pool: N(0,1) in every owned block, NaN elsewhere
    sdt = storage_dtype(dtype)
    blk_shape = (2, block_size, num_kv_heads, head_dim)
    pool = np.empty((num_blocks,) + blk_shape, dtype=sdt)
    used = np.sort(perm[:need])
    unused_mask = np.ones(num_blocks, dtype=bool)
    unused_mask[used] = False
    if fill_unused == "nan":
        pool[unused_mask] = np.float32(np.nan) if dtype == "f32" else _NAN_BITS[dtype]
    else:
        pool[unused_mask] = 0
    _fill_blocks(pool, used, seed, dtype)

    T = int(qsl[-1])
    q = _normal(rng, (T, num_q_heads, head_dim), dtype)
    k_new = _normal(rng, (T, num_kv_heads, head_dim), dtype)
    v_new = _normal(rng, (T, num_kv_heads, head_dim), dtype)

    return Workload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
        seq_lens=seq_lens, num_computed=num_computed, query_start_loc=qsl,
        block_table=table, pool=pool, q=q, k_new=k_new, v_new=v_new, seed=seed,
        meta=meta,
    )


# --------------------------------------------------------------------------
# named configurations
# --------------------------------------------------------------------------
# Llama-3-8B attention layer shape: 32 query heads, 8 KV heads (GQA 4),
# head_dim 128, block_size 16 ("vllm v1 源码精读（三）" §3.1, §3.3).

_LLAMA3 = dict(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128)


def _decode_requests(lens: Sequence[int]) -> List[Tuple[int, int]]:
    # one new token per request: it is the last of seq_len tokens
    return [(int(L) - 1, 1) for L in lens]


def _tiny_f32_decode(seed: int, values: bool = True, lens=(5, 16, 17, 100)) -> Workload:
    return build_workload(
        "tiny_f32_decode", dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=64,
        num_blocks=64, requests=_decode_requests(lens), seed=seed, table_width=7,
        scale=1.0 / 8.0, meta={"seq_lens_reading": "seq_len includes the new token"},
        values=values)


def _tiny_f32_decode_alt(seed: int, values: bool = True) -> Workload:
    w = _tiny_f32_decode(seed, values, lens=(6, 17, 18, 101))
    w.name = "tiny_f32_decode_alt"
    w.meta["seq_lens_reading"] = "context lens exclude the new token"
    return w


def _decode_bf16(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    lens = rng.integers(512, 4096, size=64, endpoint=True)
    return build_workload("decode_bf16_64req", **_LLAMA3, num_blocks=20000,
                          requests=_decode_requests(lens), seed=seed, table_width=256,
                          values=values)


def _mixed_bf16(seed: int, values: bool = True) -> Workload:
    reqs = [(1024, 512), (0, 10), (0, 10)] + [(2047, 1)] * 61
    return build_workload("mixed_chunked_prefill_bf16", **_LLAMA3, num_blocks=20000,
                          requests=reqs, seed=seed, table_width=128,
                          values=values)


def _prefill_chunk_bf16(seed: int, values: bool = True) -> Workload:
    # the mixed step's prefill chunk alone: 512 new tokens on 1024 cached
    return build_workload("prefill_chunk_bf16", **_LLAMA3, num_blocks=20000,
                          requests=[(1024, 512)], seed=seed, table_width=128,
                          values=values)


def _prefill_2k_bf16(seed: int, values: bool = True) -> Workload:
    # a 2048-token chunk on 2048 cached tokens (a token budget in the range the
    # pages advise for max_num_batched_tokens)
    return build_workload("prefill_chunk_2048_bf16", **_LLAMA3, num_blocks=20000,
                          requests=[(2048, 2048)], seed=seed, table_width=256,
                          values=values)


def _prefill_8k_bf16(seed: int, values: bool = True) -> Workload:
    # a fresh 8192-token prompt prefilled in one step
    return build_workload("prefill_8192_bf16", **_LLAMA3, num_blocks=20000,
                          requests=[(0, 8192)], seed=seed, table_width=512,
                          values=values)


def _prefill_batch_bf16(seed: int, values: bool = True) -> Workload:
    # four requests prefilling 1024-token chunks on different histories
    reqs = [(0, 1024), (1024, 1024), (3000, 1024), (512, 1000)]
    return build_workload("prefill_batch_4x1024_bf16", **_LLAMA3, num_blocks=20000,
                          requests=reqs, seed=seed, table_width=256, values=values)


def _prefix_shared_bf16(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    suffix = rng.integers(64, 512, size=256, endpoint=True)
    lens = 1024 + suffix
    return build_workload("prefix_shared_decode_bf16", **_LLAMA3, num_blocks=20000,
                          requests=_decode_requests(lens), seed=seed, table_width=96,
                          shared_prefix_blocks=64,
                          values=values)


def _long_split_bf16(seed: int, values: bool = True) -> Workload:
    return build_workload("long_context_decode_bf16", **_LLAMA3, num_blocks=36000,
                          requests=_decode_requests([32768] * 16), seed=seed,
                          table_width=2048,
                          values=values)


# ---- reduced sizes: several tiles and ragged tails, oracle finishes in seconds

def _decode_bf16_small(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    lens = list(rng.integers(1, 600, size=10, endpoint=True)) + [16, 32, 1, 17]
    return build_workload("decode_bf16_small", **_LLAMA3, num_blocks=1024,
                          requests=_decode_requests(lens), seed=seed, table_width=40,
                          values=values)


def _mixed_bf16_small(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    dec = [(int(L) - 1, 1) for L in rng.integers(1, 300, size=9, endpoint=True)]
    reqs = [(37, 100), (0, 1), (0, 10), (0, 33), (5, 0), (200, 16), (15, 17)] + dec
    return build_workload("mixed_bf16_small", **_LLAMA3, num_blocks=512,
                          requests=reqs, seed=seed, table_width=24,
                          values=values)


def _prefix_shared_small(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    lens = 64 + rng.integers(1, 80, size=16, endpoint=True)
    return build_workload("prefix_shared_small", **_LLAMA3, num_blocks=256,
                          requests=_decode_requests(lens), seed=seed, table_width=10,
                          shared_prefix_blocks=4,
                          values=values)


def _long_split_small(seed: int, values: bool = True) -> Workload:
    rng = np.random.default_rng(seed + 7_000_000)
    lens = rng.integers(3000, 5000, size=3, endpoint=True)
    return build_workload("long_decode_small", **_LLAMA3, num_blocks=1024,
                          requests=_decode_requests(lens), seed=seed, table_width=320,
                          values=values)


_BUILDERS = {
    "tiny_f32_decode": (_tiny_f32_decode, 1001),
    "tiny_f32_decode_alt": (_tiny_f32_decode_alt, 1001),
    "decode_bf16_64req": (_decode_bf16, 1002),
    "mixed_chunked_prefill_bf16": (_mixed_bf16, 1003),
    "prefix_shared_decode_bf16": (_prefix_shared_bf16, 1004),
    "prefill_chunk_bf16": (_prefill_chunk_bf16, 1006),
    "prefill_chunk_2048_bf16": (_prefill_2k_bf16, 1007),
    "prefill_8192_bf16": (_prefill_8k_bf16, 1008),
    "prefill_batch_4x1024_bf16": (_prefill_batch_bf16, 1009),
    "long_context_decode_bf16": (_long_split_bf16, 1005),
    "decode_bf16_small": (_decode_bf16_small, 2002),
    "mixed_bf16_small": (_mixed_bf16_small, 2003),
    "prefix_shared_small": (_prefix_shared_small, 2004),
    "long_decode_small": (_long_split_small, 2005),
}

CONFIG_NAMES = tuple(_BUILDERS)


def make_workload(name: str, seed: Optional[int] = None, values: bool = True) -> Workload:
    """Build the named workload; ``seed`` defaults to the config's own seed.
    ``values=False`` builds the metadata only."""
    if name not in _BUILDERS:
        raise KeyError(f"unknown workload {name!r}; known: {', '.join(CONFIG_NAMES)}")
    fn, default_seed = _BUILDERS[name]
    return fn(default_seed if seed is None else int(seed), values)
