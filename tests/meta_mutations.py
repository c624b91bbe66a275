"""Planted violations of the step metadata the kernels trust (changes to the
metadata only, made on the host), shared by the oracle's host-side check
(CPU) and the device-side check pa_check_metadata (GPU)."""

from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from workloads import make_workload


def mixed():
    return make_workload("mixed_bf16_small", values=False)


def copy_with(w, **arrays):
    return dataclasses.replace(w, **{k: np.array(v) for k, v in arrays.items()})


def slots_of(w):
    return oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, 16)


def mutations():
    """[(label, workload, slots or None, pa_check_metadata flag name)]."""
    w = mixed()
    qlen = np.diff(w.query_start_loc)
    long_r = int(np.argmax(qlen))
    out = []
    sl = w.seq_lens.copy()
    r = int(np.argmax(w.seq_lens % 16 != 0))          # a request whose last block has room
    sl[r] += 1
    out.append(("seq_len != computed + q_len", copy_with(w, seq_lens=sl), None, "computed"))
    nc = w.num_computed.copy()
    nc[0] = -1
    out.append(("negative computed", copy_with(w, num_computed=nc), None, "computed"))
    bt = w.block_table.copy()
    bt[long_r, 0] = w.num_blocks
    out.append(("block id past the pool", copy_with(w, block_table=bt), None, "block_id"))
    bt = w.block_table.copy()
    bt[long_r, 0] = -1
    out.append(("block id -1 inside seq_len", copy_with(w, block_table=bt), None, "block_id"))
    q = w.query_start_loc.copy()
    q[0] = 1
    out.append(("qsl[0] != 0", copy_with(w, query_start_loc=q), None, "query_start"))
    q = w.query_start_loc.copy()
    q[2], q[3] = q[3], q[2]
    out.append(("qsl decreasing", copy_with(w, query_start_loc=q), None, "query_start"))
    q = w.query_start_loc.copy()
    q[-1] -= 1
    out.append(("qsl[R] != T", copy_with(w, query_start_loc=q), None, "query_start"))
    bt = np.ascontiguousarray(w.block_table[:, :2])
    out.append(("table narrower than seq_len", copy_with(w, block_table=bt), None, "table_width"))
    s = slots_of(w)
    s[5] = s[6]
    out.append(("duplicate slot", w, s, "slot_dup"))
    s = slots_of(w)
    s[3] = w.num_blocks * 16
    out.append(("slot past the pool", w, s, "slot_range"))
    return out
