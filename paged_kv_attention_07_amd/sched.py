"""Python binding of the host block manager / step scheduler in libpa.so
(include/pa_sched.h).  Argument marshalling only: the scheduling runs in the
library's C++.  Step outputs land in preallocated numpy buffers (reused every
step; pass ``pin=True`` to get page-locked buffers from torch for the
host-to-device copy of the step metadata)."""

from __future__ import annotations

import ctypes
import dataclasses
from typing import List, Optional

import numpy as np

from . import PAError, lib

_i32, _i64, _u64, _sz, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t,
                              ctypes.c_void_p)


class _Config(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "num_blocks", "block_size", "max_num_batched_tokens", "max_num_seqs", "max_model_len",
        "long_prefill_token_threshold", "enable_chunked_prefill", "enable_prefix_caching")]


class _Step(ctypes.Structure):
    _fields_ = [("request_ids", _vp), ("query_start_loc", _vp), ("num_computed", _vp),
                ("seq_lens", _vp), ("block_table", _vp), ("token_ids", _vp),
                ("copy_pairs", _vp), ("preempted_ids", _vp), ("block_table_stride", _i32),
                ("num_seqs", _i32), ("num_tokens", _i32), ("max_query_len", _i32),
                ("max_seq_len", _i32), ("num_copies", _i32), ("num_preempted", _i32)]


class _Stats(ctypes.Structure):
    _fields_ = [("num_free_blocks", _i32), ("num_cached_blocks", _i32), ("num_running", _i32),
                ("num_waiting", _i32), ("num_finished", _i32), ("total_preemptions", _i64),
                ("total_prefix_hit_tokens", _i64), ("total_scheduled_tokens", _i64),
                ("total_steps", _i64)]


class _ReqInfo(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("status", "num_tokens", "num_computed", "num_generated",
                                    "num_blocks", "prompt_len")]


lib.pa_sched_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_vp)]
lib.pa_sched_create.restype = ctypes.c_int
lib.pa_sched_destroy.argtypes = [_vp]
lib.pa_sched_destroy.restype = None
lib.pa_sched_add_request.argtypes = [_vp, _i64, _vp, _i32, _i32]
lib.pa_sched_add_request.restype = ctypes.c_int
lib.pa_sched_fork.argtypes = [_vp, _i64, _i64, _i32]
lib.pa_sched_fork.restype = ctypes.c_int
lib.pa_sched_schedule.argtypes = [_vp, ctypes.POINTER(_Step)]
lib.pa_sched_schedule.restype = ctypes.c_int
lib.pa_sched_update.argtypes = [_vp, _vp, _i32, _vp, ctypes.POINTER(_i32)]
lib.pa_sched_update.restype = ctypes.c_int
lib.pa_sched_get_stats.argtypes = [_vp, ctypes.POINTER(_Stats)]
lib.pa_sched_get_stats.restype = ctypes.c_int
lib.pa_sched_get_request.argtypes = [_vp, _i64, ctypes.POINTER(_ReqInfo), _vp, _i32]
lib.pa_sched_get_request.restype = ctypes.c_int
lib.pa_sched_get_free_queue.argtypes = [_vp, _vp, _i32, ctypes.POINTER(_i32)]
lib.pa_sched_get_free_queue.restype = ctypes.c_int
lib.pa_sched_get_block.argtypes = [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_u64),
                                   ctypes.POINTER(_i32)]
lib.pa_sched_get_block.restype = ctypes.c_int
lib.pa_xxh64.argtypes = [_vp, _sz, _u64]
lib.pa_xxh64.restype = _u64
lib.pa_block_hash.argtypes = [_u64, _i32, _vp, _i32]
lib.pa_block_hash.restype = _u64

STATUS = {0: "waiting", 1: "running", 2: "finished"}


def _check(fn: str, st: int) -> int:
    if st < 0:
        raise PAError(fn, st)
    return st


def xxh64(data: bytes, seed: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    return lib.pa_xxh64(buf, len(data), seed)


def block_hash(parent: Optional[int], tokens) -> int:
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return lib.pa_block_hash(0 if parent is None else parent, parent is not None,
                             t.ctypes.data, t.size)


@dataclasses.dataclass
class Step:
    """Views of one step's metadata (valid until the same buffer set is
    reused, two schedule() calls later)."""
    request_ids: np.ndarray
    query_start_loc: np.ndarray
    num_computed: np.ndarray
    seq_lens: np.ndarray
    block_table: np.ndarray          # [num_seqs, stride]
    token_ids: np.ndarray
    copy_pairs: np.ndarray           # [num_copies, 2]
    preempted: np.ndarray
    max_query_len: int
    max_seq_len: int
    buffer: int                      # which buffer set holds it
    arena_len: int                   # int32 elements of the arena in use

    @property
    def num_seqs(self) -> int:
        return int(self.request_ids.size)

    @property
    def num_tokens(self) -> int:
        return int(self.token_ids.size)

    @property
    def num_new(self) -> np.ndarray:
        return np.diff(self.query_start_loc)


class ArenaLayout:
    """One int32 arena per buffer set holding everything the GPU needs, so a
    step's metadata goes to the device in one copy of its used prefix:
    [query_start_loc S+1 | num_computed S | seq_lens S | copy_pairs 2S |
     block_table S x stride]."""

    def __init__(self, max_num_seqs: int, stride: int):
        S = max_num_seqs
        self.S, self.stride = S, stride
        self.qsl = 0
        self.nc = S + 1
        self.sl = 2 * S + 1
        self.cp = 3 * S + 1
        self.bt = 5 * S + 1
        self.size = self.bt + S * stride

    def used(self, num_seqs: int) -> int:
        return self.bt + num_seqs * self.stride


class Scheduler:
    def __init__(self, num_blocks: int, block_size: int, max_num_batched_tokens: int,
                 max_num_seqs: int, max_model_len: int, enable_chunked_prefill: bool = True,
                 enable_prefix_caching: bool = True, long_prefill_token_threshold: int = 0,
                 pin: bool = False, num_buffers: int = 2):
        cfg = _Config(num_blocks, block_size, max_num_batched_tokens, max_num_seqs,
                      max_model_len, long_prefill_token_threshold, int(enable_chunked_prefill),
                      int(enable_prefix_caching))
        h = _vp()
        _check("pa_sched_create", lib.pa_sched_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_num_seqs = max_num_seqs
        self.stride = -(-max_model_len // block_size)
        self.layout = L = ArenaLayout(max_num_seqs, self.stride)
        S, T = max_num_seqs, max_num_batched_tokens
        # arenas: torch pinned tensors when pin=True (kept so copies from
        # them are asynchronous), numpy views either way
        self.arenas_torch, self.arenas = [], []
        for _ in range(num_buffers):
            if pin:
                import torch
                t = torch.empty(L.size, dtype=torch.int32, pin_memory=True)
                self.arenas_torch.append(t)
                self.arenas.append(t.numpy())
            else:
                self.arenas.append(np.empty(L.size, np.int32))
        self._ids = [np.empty(S, np.int64) for _ in range(num_buffers)]
        self._pre = [np.empty(S, np.int64) for _ in range(num_buffers)]
        self._tok = [np.empty(T, np.int32) for _ in range(num_buffers)]
        self._steps = []
        for i, a in enumerate(self.arenas):
            base = a.ctypes.data
            self._steps.append(_Step(
                self._ids[i].ctypes.data, base + 4 * L.qsl, base + 4 * L.nc, base + 4 * L.sl,
                base + 4 * L.bt, self._tok[i].ctypes.data, base + 4 * L.cp,
                self._pre[i].ctypes.data, self.stride, 0, 0, 0, 0, 0, 0))
        self._next = 0
        self._finished = np.empty(S, np.int64)

    @classmethod
    def view(cls, handle) -> "Scheduler":
        """A non-owning handle on a scheduler created elsewhere (an engine's):
        requests, forks and inspection only."""
        self = cls.__new__(cls)
        self._h, self._owned, self._steps = handle, False, []
        return self

    def close(self) -> None:
        if self._h and getattr(self, "_owned", True):
            lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- requests
    def add_request(self, request_id: int, prompt, max_new_tokens: int) -> None:
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        _check("pa_sched_add_request",
               lib.pa_sched_add_request(self._h, request_id, p.ctypes.data, p.size,
                                        max_new_tokens))

    def fork(self, parent_id: int, child_id: int, max_new_tokens: int) -> bool:
        return bool(_check("pa_sched_fork",
                           lib.pa_sched_fork(self._h, parent_id, child_id, max_new_tokens)))

    # ---- steps
    def schedule(self) -> Step:
        i = self._next
        self._next = (i + 1) % len(self._steps)
        st = self._steps[i]
        _check("pa_sched_schedule", lib.pa_sched_schedule(self._h, ctypes.byref(st)))
        a, L, n = self.arenas[i], self.layout, st.num_seqs
        return Step(request_ids=self._ids[i][:n], query_start_loc=a[L.qsl:L.qsl + n + 1],
                    num_computed=a[L.nc:L.nc + n], seq_lens=a[L.sl:L.sl + n],
                    block_table=a[L.bt:L.bt + n * self.stride].reshape(n, self.stride),
                    token_ids=self._tok[i][:st.num_tokens],
                    copy_pairs=a[L.cp:L.cp + 2 * st.num_copies].reshape(-1, 2),
                    preempted=self._pre[i][:st.num_preempted],
                    max_query_len=st.max_query_len, max_seq_len=st.max_seq_len,
                    buffer=i, arena_len=L.used(n))

    def update(self, sampled) -> List[int]:
        s = np.ascontiguousarray(sampled, dtype=np.int32)
        nf = _i32()
        _check("pa_sched_update", lib.pa_sched_update(self._h, s.ctypes.data, s.size,
                                                      self._finished.ctypes.data,
                                                      ctypes.byref(nf)))
        return [int(x) for x in self._finished[:nf.value]]

    # ---- inspection
    def stats(self) -> dict:
        st = _Stats()
        _check("pa_sched_get_stats", lib.pa_sched_get_stats(self._h, ctypes.byref(st)))
        return {k: getattr(st, k) for k, _ in _Stats._fields_}

    def request(self, request_id: int) -> dict:
        info = _ReqInfo()
        _check("pa_sched_get_request", lib.pa_sched_get_request(
            self._h, request_id, ctypes.byref(info), None, 0))
        blocks = np.empty(max(info.num_blocks, 1), np.int32)
        _check("pa_sched_get_request", lib.pa_sched_get_request(
            self._h, request_id, ctypes.byref(info), blocks.ctypes.data, blocks.size))
        d = {k: getattr(info, k) for k, _ in _ReqInfo._fields_}
        d["status"] = STATUS[d["status"]]
        d["blocks"] = blocks[:info.num_blocks].tolist()
        return d

    def free_queue(self) -> List[int]:
        n = _i32()
        _check("pa_sched_get_free_queue", lib.pa_sched_get_free_queue(
            self._h, None, 0, ctypes.byref(n)))
        out = np.empty(max(n.value, 1), np.int32)
        _check("pa_sched_get_free_queue", lib.pa_sched_get_free_queue(
            self._h, out.ctypes.data, out.size, ctypes.byref(n)))
        return out[:n.value].tolist()

    def block(self, block_id: int):
        r, h, has = _i32(), _u64(), _i32()
        _check("pa_sched_get_block", lib.pa_sched_get_block(
            self._h, block_id, ctypes.byref(r), ctypes.byref(h), ctypes.byref(has)))
        return r.value, (h.value if has.value else None)
