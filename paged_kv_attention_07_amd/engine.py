"""Python binding of the multi-step driver (include/pa_engine.h): the
library's C++ scheduler plans each step and the same native call launches
the metadata copy, block copies, slot mapping, K/V scatter and attention on
the current stream.  This module only marshals arguments and owns the device
buffers (KV cache, scratch, output) as torch tensors."""

from __future__ import annotations

import ctypes
from typing import List, Optional

import numpy as np

from . import DTYPE_CODES, PAError, _dev, _stream, lib
from .sched import Scheduler, Step, _Config, _Step

_i32, _i64, _sz, _f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float,
                              ctypes.c_void_p)


class _Geometry(ctypes.Structure):
    _fields_ = [("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("dtype", _i32), ("scale", _f32), ("num_splits", _i32)]


lib.pa_engine_device_bytes.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Geometry)]
lib.pa_engine_device_bytes.restype = _sz
lib.pa_engine_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Geometry), _vp, _vp,
                                 _sz, ctypes.POINTER(_vp)]
lib.pa_engine_create.restype = ctypes.c_int
lib.pa_engine_destroy.argtypes = [_vp]
lib.pa_engine_destroy.restype = None
lib.pa_engine_scheduler.argtypes = [_vp]
lib.pa_engine_scheduler.restype = _vp
lib.pa_engine_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_Step)]
lib.pa_engine_step.restype = ctypes.c_int
lib.pa_engine_update.argtypes = [_vp, _vp, _i32, _vp, ctypes.POINTER(_i32)]
lib.pa_engine_update.restype = ctypes.c_int


def _arr(ptr, n, ctype, dt):
    if n <= 0 or not ptr:
        return np.empty(0, dt)
    return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctype)), shape=(n,))


class Engine:
    def __init__(self, *, num_blocks: int, max_num_batched_tokens: int, max_num_seqs: int,
                 max_model_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 dtype: str = "bf16", block_size: int = 16, enable_chunked_prefill: bool = True,
                 enable_prefix_caching: bool = True, long_prefill_token_threshold: int = 0,
                 num_splits: int = 0, scale: Optional[float] = None):
        import torch
        self.torch = torch
        self.cfg = _Config(num_blocks, block_size, max_num_batched_tokens, max_num_seqs,
                           max_model_len, long_prefill_token_threshold,
                           int(enable_chunked_prefill), int(enable_prefix_caching))
        self.scale = float(scale if scale is not None else head_dim ** -0.5)
        self.geo = _Geometry(num_q_heads, num_kv_heads, head_dim, DTYPE_CODES[dtype],
                             self.scale, num_splits)
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        self.dtype, self.T = dtype, max_num_batched_tokens
        nbytes = lib.pa_engine_device_bytes(ctypes.byref(self.cfg), ctypes.byref(self.geo))
        if nbytes == 0:
            raise ValueError("unsupported engine configuration")
        dev = torch.device("cuda")
        self.kv = torch.empty((num_blocks, 2, block_size, num_kv_heads, head_dim), dtype=tdt,
                              device=dev)
        self.scratch = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((max_num_batched_tokens, num_q_heads, head_dim), dtype=tdt,
                               device=dev)
        h = _vp()
        st = lib.pa_engine_create(ctypes.byref(self.cfg), ctypes.byref(self.geo),
                                  self.kv.data_ptr(), self.scratch.data_ptr(), nbytes,
                                  ctypes.byref(h))
        if st != 0:
            raise PAError("pa_engine_create", st)
        self._h = h
        self.sched = Scheduler.view(lib.pa_engine_scheduler(h))
        self._step = _Step()
        self._views = {}
        self._finished = np.empty(max_num_seqs, np.int64)
        self._stride = -(-max_model_len // block_size)

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib.pa_engine_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- requests
    def add_request(self, request_id: int, prompt, max_new_tokens: int) -> None:
        self.sched.add_request(request_id, prompt, max_new_tokens)

    def fork(self, parent_id: int, child_id: int, max_new_tokens: int) -> bool:
        return self.sched.fork(parent_id, child_id, max_new_tokens)

    # ---- one step
    def step(self, q, k, v) -> Step:
        """Plan and launch one step on the current stream.  q [>= T, Hq, D],
        k / v [>= T, Hkv, D]; the attention output is self.out[:num_tokens]."""
        s = self._step
        st = lib.pa_engine_step(self._h, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                self.out.data_ptr(), _stream(), ctypes.byref(s))
        if st != 0:
            raise PAError("pa_engine_step", st)
        n = s.num_seqs
        v = self._views.get(s.request_ids)
        if v is None:
            # full-capacity views of this arena set, built once (the engine's
            # arenas never move)
            S, T, W = len(self._finished), self.T, self._stride
            v = self._views[s.request_ids] = dict(
                ids=_arr(s.request_ids, S, ctypes.c_int64, np.int64),
                qsl=_arr(s.query_start_loc, S + 1, ctypes.c_int32, np.int32),
                nc=_arr(s.num_computed, S, ctypes.c_int32, np.int32),
                sl=_arr(s.seq_lens, S, ctypes.c_int32, np.int32),
                bt=_arr(s.block_table, S * W, ctypes.c_int32, np.int32).reshape(S, W),
                tok=_arr(s.token_ids, T, ctypes.c_int32, np.int32),
                cp=_arr(s.copy_pairs, 2 * S, ctypes.c_int32, np.int32).reshape(S, 2),
                pre=_arr(s.preempted_ids, S, ctypes.c_int64, np.int64))
        return Step(request_ids=v["ids"][:n], query_start_loc=v["qsl"][:n + 1],
                    num_computed=v["nc"][:n], seq_lens=v["sl"][:n], block_table=v["bt"][:n],
                    token_ids=v["tok"][:s.num_tokens], copy_pairs=v["cp"][:s.num_copies],
                    preempted=v["pre"][:s.num_preempted], max_query_len=s.max_query_len,
                    max_seq_len=s.max_seq_len, buffer=-1, arena_len=0)

    def update(self, sampled) -> List[int]:
        smp = np.ascontiguousarray(sampled, dtype=np.int32)
        nf = _i32()
        st = lib.pa_engine_update(self._h, smp.ctypes.data, smp.size, self._finished.ctypes.data,
                                  ctypes.byref(nf))
        if st != 0:
            raise PAError("pa_engine_update", st)
        return [int(x) for x in self._finished[:nf.value]]

    def stats(self) -> dict:
        return self.sched.stats()
