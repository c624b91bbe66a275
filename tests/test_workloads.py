"""The seeded input generators: shapes, lengths and table structure of every
named workload match the configurations they stand for."""

import numpy as np
import pytest

import oracle
from workloads import CONFIG_NAMES, make_workload

BIG = {"decode_bf16_64req", "mixed_chunked_prefill_bf16", "prefix_shared_decode_bf16",
       "long_context_decode_bf16", "prefill_chunk_2048_bf16", "prefill_8192_bf16",
       "prefill_batch_4x1024_bf16", "prefill_chunk_bf16"}


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_metadata_consistent(name):
    w = make_workload(name, values=False)
    B = w.block_size
    oracle.validate_metadata(w.block_table, w.seq_lens, w.query_start_loc, w.num_computed,
                             w.num_blocks, B)
    # table entries beyond ceil(L/B) are -1; within, ids are in range
    for r in range(w.num_seqs):
        nb = oracle.blocks_for_tokens(int(w.seq_lens[r]), B)
        assert np.all(w.block_table[r, nb:] == -1)
    # slots of this step's tokens are distinct (the scatter's precondition)
    slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, B)
    assert np.unique(slots).size == slots.size
    # deterministic
    w2 = make_workload(name, values=False)
    assert np.array_equal(w.block_table, w2.block_table)
    assert np.array_equal(w.seq_lens, w2.seq_lens)


def test_config_shapes():
    c1 = make_workload("tiny_f32_decode", values=False)
    assert list(c1.seq_lens) == [5, 16, 17, 100] and c1.dtype == "f32"
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.num_blocks) == (4, 2, 64, 64)
    assert c1.scale == 1.0 / 8.0 and c1.is_decode_only
    c2 = make_workload("decode_bf16_64req", values=False)
    assert c2.num_seqs == 64 and c2.seq_lens.min() >= 512 and c2.seq_lens.max() <= 4096
    assert (c2.num_q_heads, c2.num_kv_heads, c2.head_dim, c2.num_blocks) == (32, 8, 128, 20000)
    c3 = make_workload("mixed_chunked_prefill_bf16", values=False)
    assert c3.num_seqs == 64 and c3.num_tokens == 593
    assert list(c3.q_lens[:3]) == [512, 10, 10] and np.all(c3.q_lens[3:] == 1)
    assert c3.seq_lens[0] == 1536 and np.all(c3.seq_lens[3:] == 2048)
    c4 = make_workload("prefix_shared_decode_bf16", values=False)
    assert c4.num_seqs == 256
    assert np.all(c4.block_table[:, :64] == c4.block_table[0, :64])
    suffix = c4.seq_lens - 1024
    assert suffix.min() >= 64 and suffix.max() <= 512
    private = np.concatenate([c4.block_table[r, 64:oracle.blocks_for_tokens(int(L), 16)]
                              for r, L in enumerate(c4.seq_lens)])
    assert np.unique(private).size == private.size
    assert not np.isin(private, c4.block_table[0, :64]).any()
    c5 = make_workload("long_context_decode_bf16", values=False)
    assert c5.num_seqs == 16 and np.all(c5.seq_lens == 32768) and c5.num_blocks == 36000
    ids = c5.block_table[c5.block_table >= 0]
    assert ids.size == 16 * 2048 and np.unique(ids).size == ids.size
    # the pool is larger than 2^31 bytes: offsets must be 64-bit
    assert c5.num_blocks * oracle.block_bytes(16, 8, 128, 2) > 2 ** 31
    c6 = make_workload("prefill_chunk_2048_bf16", values=False)
    assert list(c6.q_lens) == [2048] and list(c6.num_computed) == [2048]
    c7 = make_workload("prefill_8192_bf16", values=False)
    assert list(c7.q_lens) == [8192] and list(c7.num_computed) == [0]
    c8 = make_workload("prefill_batch_4x1024_bf16", values=False)
    assert list(c8.q_lens) == [1024, 1024, 1024, 1000]
    assert list(c8.seq_lens) == [1024, 2048, 4024, 1512]


@pytest.mark.parametrize("name", [n for n in CONFIG_NAMES if n not in BIG])
def test_values(name):
    w = make_workload(name)
    assert w.pool.shape == (w.num_blocks, 2, w.block_size, w.num_kv_heads, w.head_dim)
    assert w.pool.strides[0] == oracle.block_bytes(w.block_size, w.num_kv_heads, w.head_dim,
                                                   w.pool.itemsize)
    assert w.q.shape == (w.num_tokens, w.num_q_heads, w.head_dim)
    vals = oracle.decode_bits(w.pool, w.dtype)
    used = np.zeros(w.num_blocks, bool)
    used[w.used_blocks] = True
    assert np.all(np.isnan(vals[~used]))
    assert np.all(np.isfinite(vals[used]))
    qv = oracle.decode_bits(w.q, w.dtype)
    assert abs(qv.mean()) < 0.1 and 0.9 < qv.std() < 1.1
