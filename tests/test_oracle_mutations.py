"""Plant plausible mistakes in the oracle (on the CPU) and require that the
pins catch each one: a pin set that passes a broken oracle proves nothing."""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import ref


def _bad_gqa(h, group):           # query head -> wrong KV head (interleaved groups)
    return h % max(1, group)


def _bad_causal_strict(pos, j):   # drops the query's own key
    return j < pos


def _bad_causal_none(pos, j):     # no causal mask inside a chunk
    return j >= 0


def _bad_softmax_sign(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(m - s)
    e = np.where(np.isfinite(s), e, 0.0)
    return e / np.sum(e, axis=-1, keepdims=True)


def _bad_scores_no_scale(q_rows, K_head, scale):
    return q_rows @ K_head.T


def _bad_scores_transposed(q_rows, K_head, scale):
    D = q_rows.shape[1]
    return scale * (q_rows.reshape(-1, D)[:, ::-1] @ K_head.T)


def _bad_offset(pos, block_size):
    return (pos + 1) % block_size


def _bad_logical(pos, block_size):
    return pos % block_size if pos % block_size < 3 else pos // block_size


_orig_gather = ref.gather_request_kv


def _bad_gather_swap(pool, row, L, dtype):
    K, V = _orig_gather(pool, row, L, dtype)
    return V, K


def _bad_gather_reversed_blocks(pool, row, L, dtype):
    nb = -(-L // pool.shape[2])
    rev = np.array(row, copy=True)
    rev[:nb] = rev[:nb][::-1]
    return _orig_gather(pool, rev, L, dtype)


def _bad_merge(m, l, o):
    M = np.max(m)
    w = np.exp(M - m)
    return (w[:, None] * o).sum(axis=0) / np.sum(w * l)


_orig_decode = ref.decode_bits


def _bad_decode(a, dtype):
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return u.view(np.float32).astype(np.float64)
    return _orig_decode(a, dtype)


def _bad_kv_bytes(num_kv_heads, head_dim, elem_bytes, num_layers=1):
    return num_kv_heads * head_dim * elem_bytes * num_layers


_orig_rac = ref.reshape_and_cache


def _bad_rac_kv_swapped(pool, key, value, slots):
    return _orig_rac(pool, value, key, slots)


_orig_copy = ref.copy_blocks


def _bad_copy_k_only(pool, pairs):
    out = _orig_copy(pool, pairs)
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        if src >= 0 and dst >= 0:
            out[dst, 1] = pool[dst, 1]
    return out


def _bad_copy_reversed(pool, pairs):
    p = np.asarray(pairs).reshape(-1, 2)
    out = pool.copy()
    for src, dst in p:
        if src >= 0 and dst >= 0:
            out[src] = pool[dst]
    return out


_orig_mask = ref.used_slot_mask


def _bad_mask_extra(block_table, seq_lens, num_blocks, block_size):
    # one position past each request's end also marked
    return _orig_mask(block_table, np.asarray(seq_lens) + 1, num_blocks, block_size)


def _bad_mask_short(block_table, seq_lens, num_blocks, block_size):
    return _orig_mask(block_table, np.maximum(np.asarray(seq_lens) - 1, 0), num_blocks,
                      block_size)


_orig_validate = ref.validate_metadata


def _bad_validate_no_ids(block_table, seq_lens, query_start_loc, num_computed, num_blocks,
                         block_size, slots=None):
    # block ids not checked: a wide pool makes every id valid
    return _orig_validate(np.abs(block_table), seq_lens, query_start_loc, num_computed,
                          1 << 30, block_size, slots)


def _bad_validate_no_slots(block_table, seq_lens, query_start_loc, num_computed, num_blocks,
                           block_size, slots=None):
    return _orig_validate(block_table, seq_lens, query_start_loc, num_computed, num_blocks,
                          block_size, None)


MUTATIONS = {
    "gqa_interleaved": ("kv_head_of", _bad_gqa),
    "causal_strict": ("visible", _bad_causal_strict),
    "causal_missing": ("visible", _bad_causal_none),
    "softmax_sign": ("_softmax_rows", _bad_softmax_sign),
    "scale_dropped": ("scores", _bad_scores_no_scale),
    "operand_reversed": ("scores", _bad_scores_transposed),
    "slot_offset_off_by_one": ("offset_in_block", _bad_offset),
    "slot_block_index": ("logical_block_of", _bad_logical),
    "k_v_swapped_on_read": ("gather_request_kv", _bad_gather_swap),
    "block_order_reversed": ("gather_request_kv", _bad_gather_reversed_blocks),
    "merge_weight_sign": ("merge_partials", _bad_merge),
    "bf16_decode_shift": ("decode_bits", _bad_decode),
    "kv_bytes_missing_factor_2": ("kv_bytes_per_token", _bad_kv_bytes),
    "k_v_swapped_on_write": ("reshape_and_cache", _bad_rac_kv_swapped),
    "copy_blocks_k_only": ("copy_blocks", _bad_copy_k_only),
    "copy_blocks_direction": ("copy_blocks", _bad_copy_reversed),
    "used_slot_mask_one_past_end": ("used_slot_mask", _bad_mask_extra),
    "used_slot_mask_one_short": ("used_slot_mask", _bad_mask_short),
    "validate_ignores_block_ids": ("validate_metadata", _bad_validate_no_ids),
    "validate_ignores_slots": ("validate_metadata", _bad_validate_no_slots),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    import oracle
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(ref, attr, bad)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, bad)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except Exception as e:  # AssertionError or a crash both count
            caught.append(check.__name__)
    assert caught, f"mutation {name} passed every pin"
