"""Plain fp64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the HIP library or its binding.

Sources (web pages, cited by title and section):
  [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成"
  [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
  [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"

What is computed.  Paging is only addressing: the result is, for every query
token, exact softmax attention over its own request's keys 0..pos, where pos
is the token's absolute position ([P2] §3.4 step 3: each sequence attends only
to its own tokens; [P4] §4.2: a prefill chunk attends its cached history plus
the earlier tokens of the chunk, a decode token attends all its history).
The oracle gathers K/V through the block table and writes that definition out
in float64.  Readings of points the pages leave open:
  * seq_lens[r] counts every key the request's last query sees, including the
    tokens written this step ([P4] §4.2: a decode request with 754 cached
    tokens attends 755 keys);
  * GQA query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * scale is an argument (1/sqrt(head_dim) in [P1] §4.2's sketch);
  * a negative slot means "padding token, write nothing";
  * slots not covered by a request's 0..seq_len-1 positions are never read.
"""

from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# element decoding
# --------------------------------------------------------------------------


def decode_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits -> float64.  bf16 is the top half of an IEEE float32."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# sizes ([P4] §3.1, [P2] §3.1, [P1] §4.2, [P2] §3.3)
# --------------------------------------------------------------------------


def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int,
                       num_layers: int = 1) -> int:
    """K and V of one token: 2 x kv heads x head_dim x element bytes per layer ([P4] §3.1)."""
    return 2 * num_kv_heads * head_dim * elem_bytes * num_layers


def block_bytes(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int,
                num_layers: int = 1) -> int:
    """One paged block: 2 x block_size x kv heads x head_size x dtype bytes ([P2] §3.1)."""
    return 2 * block_size * num_kv_heads * head_dim * elem_bytes * num_layers


def blocks_for_tokens(n: int, block_size: int) -> int:
    """Blocks needed for n tokens: ceil(n / block_size) ([P2] §3.3, allocate_slots)."""
    return -(-int(n) // int(block_size))


# --------------------------------------------------------------------------
# addressing ([P4] §3.4)
# --------------------------------------------------------------------------


def logical_block_of(pos: int, block_size: int) -> int:
    return pos // block_size


def offset_in_block(pos: int, block_size: int) -> int:
    return pos % block_size


def slot_of(block_table: np.ndarray, r: int, pos: int, block_size: int) -> int:
    """Physical slot of request r's token at absolute position pos ([P4] §3.4):
    the logical block pos // B is looked up in the request's table row, and the
    slot is that physical block id times B plus the offset pos % B."""
    phys = int(block_table[r, logical_block_of(pos, block_size)])
    if phys < 0:
        raise ValueError(f"request {r} position {pos}: block table entry is -1")
    return phys * block_size + offset_in_block(pos, block_size)


def slot_mapping(block_table: np.ndarray, query_start_loc: np.ndarray,
                 num_computed: np.ndarray, block_size: int) -> np.ndarray:
    """Slot of every query token of the step, in varlen order ([P4] §3.4:
    one 1-D entry per token, aligned with the packed input ids).  Token i of
    request r sits at position num_computed[r] + i ([P1] §3.3.2, positions)."""
    T = int(query_start_loc[-1])
    out = np.empty(T, dtype=np.int64)
    for r in range(len(num_computed)):
        t0, t1 = int(query_start_loc[r]), int(query_start_loc[r + 1])
        for i in range(t1 - t0):
            out[t0 + i] = slot_of(block_table, r, int(num_computed[r]) + i, block_size)
    return out


def used_slot_mask(block_table: np.ndarray, seq_lens: np.ndarray, num_blocks: int,
                   block_size: int) -> np.ndarray:
    """[num_blocks, block_size] mask of slots that hold one of a request's
    positions 0..seq_len-1 (the only slots attention may read)."""
    m = np.zeros((num_blocks, block_size), dtype=bool)
    for r, L in enumerate(seq_lens):
        for pos in range(int(L)):
            s = slot_of(block_table, r, pos, block_size)
            m[s // block_size, s % block_size] = True
    return m


# --------------------------------------------------------------------------
# write path: reshape_and_cache ([P1] §3.3.3, [P4] §3.4)
# --------------------------------------------------------------------------


def reshape_and_cache(pool: np.ndarray, key: np.ndarray, value: np.ndarray,
                      slots: np.ndarray) -> np.ndarray:
    """Return a copy of the pool with token t's key and value rows stored at
    slot slots[t]: K half (index 0) and V half (index 1) of block s // B at
    offset s % B.  Bits are copied unchanged; slot < 0 writes nothing."""
    out = pool.copy()
    B = pool.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = int(s) // B, int(s) % B
        if blk >= pool.shape[0]:
            raise IndexError(f"slot {int(s)} beyond the pool")
        out[blk, 0, off] = key[t]
        out[blk, 1, off] = value[t]
    return out


def copy_blocks(pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """Copy-on-write block fork ([P1] §4.3.2: samples of one prompt share its
    blocks; a sample about to write into a shared block gets a private copy).
    Return a copy of the pool where, for every (src, dst) row of `pairs`,
    block dst holds block src's K and V bits.  A row with a negative entry is
    skipped.  Precondition (the library's too): destinations are distinct and
    none of them is also a source in the same call, so the order of the
    copies does not matter."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    live = pairs[(pairs[:, 0] >= 0) & (pairs[:, 1] >= 0)]
    if np.unique(live[:, 1]).size != live.shape[0]:
        raise ValueError("copy_blocks: destinations must be distinct")
    if np.isin(live[:, 1], live[:, 0]).any():
        raise ValueError("copy_blocks: a destination is also a source")
    if live.size and live.max() >= pool.shape[0]:
        raise IndexError("copy_blocks: block id beyond the pool")
    out = pool.copy()
    for src, dst in live:
        out[dst] = pool[src]
    return out


# --------------------------------------------------------------------------
# read path: paged attention ([P1] §3.3.3 / §4.2, [P2] §3.4, [P4] §3.4 / §4.2)
# --------------------------------------------------------------------------


def kv_head_of(h: int, group: int) -> int:
    """GQA: query head h shares KV head h // group (group = Hq / Hkv)."""
    return h // group


def visible(pos: int, j: np.ndarray) -> np.ndarray:
    """Causal rule: the query at absolute position pos sees keys j <= pos."""
    return j <= pos


def gather_request_kv(pool: np.ndarray, table_row: np.ndarray, seq_len: int,
                      dtype: str) -> Tuple[np.ndarray, np.ndarray]:
    """K, V of positions 0..seq_len-1 of one request as float64 [L, Hkv, D]:
    position j lives in physical block table_row[j // B] at offset j % B."""
    B = pool.shape[2]
    nb = blocks_for_tokens(seq_len, B)
    blocks = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and (blocks.min() < 0 or blocks.max() >= pool.shape[0]):
        raise IndexError("block table entry out of range")
    Hkv, D = pool.shape[3], pool.shape[4]
    K = pool[blocks, 0].reshape(nb * B, Hkv, D)[:seq_len]
    V = pool[blocks, 1].reshape(nb * B, Hkv, D)[:seq_len]
    return decode_bits(K, dtype), decode_bits(V, dtype)


def scores(q_rows: np.ndarray, K_head: np.ndarray, scale: float) -> np.ndarray:
    """s[i, j] = scale * <q_i, K_j> for query rows [n, D] and keys [L, D]."""
    return scale * (q_rows @ K_head.T)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def paged_attention(q: np.ndarray, pool: np.ndarray, block_table: np.ndarray,
                    seq_lens: np.ndarray, query_start_loc: np.ndarray,
                    num_computed: np.ndarray, scale: float, dtype: str,
                    requests: Sequence[int] = None) -> np.ndarray:
    """Attention output [T, Hq, D] in float64 for the packed queries ``q``.

    For request r and its i-th query of this step: t = query_start_loc[r] + i,
    pos = num_computed[r] + i; scores s_j = scale * <q[t, h], K_j[h // G]> for
    keys j = 0..pos; out[t, h] = sum_j softmax(s)_j V_j[h // G].
    Decode is the case of one query at pos = seq_len - 1.  ``requests``
    restricts the work to a subset (other rows stay NaN)."""
    T, Hq, D = q.shape
    Hkv = pool.shape[3]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    qf = decode_bits(q, dtype)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    rs = range(len(seq_lens)) if requests is None else requests
    for r in rs:
        t0, t1 = int(query_start_loc[r]), int(query_start_loc[r + 1])
        n = t1 - t0
        if n == 0:
            continue
        L = int(seq_lens[r])
        c = int(num_computed[r])
        if c + n != L:
            raise ValueError(f"request {r}: num_computed + q_len != seq_len")
        K, V = gather_request_kv(pool, block_table[r], L, dtype)
        j = np.arange(L)
        mask = np.stack([visible(c + i, j) for i in range(n)])      # [n, L]
        for h in range(Hq):
            g = kv_head_of(h, G)
            s = scores(qf[t0:t1, h, :], K[:, g, :], scale)           # [n, L]
            s = np.where(mask, s, -np.inf)
            p = _softmax_rows(s)
            out[t0:t1, h, :] = p @ V[:, g, :]
    return out


# --------------------------------------------------------------------------
# split-KV partial results and their merge (online-softmax identity,
# [P1] §6.4 "Online Softmax"; partition-and-reduce for long contexts)
# --------------------------------------------------------------------------


def paged_attention_partials(q_row: np.ndarray, K: np.ndarray, V: np.ndarray,
                             scale: float, partition: int):
    """For one query vector and one head's keys [L, D], per partition p of
    ``partition`` consecutive keys: m_p = max score, l_p = sum exp(s - m_p),
    o_p = sum exp(s - m_p) V (unnormalised)."""
    L = K.shape[0]
    ms, ls, os_ = [], [], []
    for a in range(0, L, partition):
        s = scale * (K[a:a + partition] @ q_row)
        m = np.max(s)
        e = np.exp(s - m)
        ms.append(m)
        ls.append(np.sum(e))
        os_.append(e @ V[a:a + partition])
    return np.array(ms), np.array(ls), np.array(os_)


def merge_partials(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Combine partitions: M = max_p m_p, out = sum_p e^(m_p-M) o_p / sum_p e^(m_p-M) l_p."""
    M = np.max(m)
    w = np.exp(m - M)
    return (w[:, None] * o).sum(axis=0) / np.sum(w * l)


# --------------------------------------------------------------------------
# chunked prefill: token budget split of a prompt ([P4] §4.2)
# --------------------------------------------------------------------------


def chunk_schedule(prompt_len: int, budget: int) -> List[int]:
    """Chunk sizes a prompt is prefilled in when each step grants ``budget``
    tokens: num_new = min(remaining, budget) until nothing remains."""
    sizes, remaining = [], int(prompt_len)
    while remaining > 0:
        n = min(remaining, int(budget))
        sizes.append(n)
        remaining -= n
    return sizes


# --------------------------------------------------------------------------
# metadata checks (preconditions the kernels trust)
# --------------------------------------------------------------------------


def validate_metadata(block_table: np.ndarray, seq_lens: np.ndarray,
                      query_start_loc: np.ndarray, num_computed: np.ndarray,
                      num_blocks: int, block_size: int,
                      slots: np.ndarray = None) -> None:
    R = len(seq_lens)
    if query_start_loc.shape != (R + 1,) or int(query_start_loc[0]) != 0:
        raise ValueError("query_start_loc must be [R+1] starting at 0")
    qlen = np.diff(query_start_loc)
    if np.any(qlen < 0):
        raise ValueError("query_start_loc must be non-decreasing")
    if np.any(num_computed + qlen != seq_lens):
        raise ValueError("seq_lens must equal num_computed + q_len")
    if np.any(num_computed < 0):
        raise ValueError("negative num_computed")
    for r in range(R):
        nb = blocks_for_tokens(int(seq_lens[r]), block_size)
        if nb > block_table.shape[1]:
            raise ValueError(f"request {r}: table too narrow")
        ids = block_table[r, :nb]
        if np.any(ids < 0) or np.any(ids >= num_blocks):
            raise ValueError(f"request {r}: block id out of range")
    if slots is not None:
        s = np.asarray(slots)
        s = s[s >= 0]
        if np.unique(s).size != s.size:
            raise ValueError("duplicate slots in one call")
        if s.size and int(s.max()) >= num_blocks * block_size:
            raise ValueError("slot beyond the pool")
