"""Paged KV attention on MI355X (gfx950): Python binding of libpa.so.

The functions here only marshal arguments: they check tensor metadata,
allocate outputs / workspace with torch (device memory plumbing) and call the
C ABI declared in include/pa.h on torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
If libpa.so has not been built, importing this package raises ImportError.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PAError", "lib", "library_path", "DTYPE_CODES",
    "pa_compute_slot_mapping", "pa_reshape_and_cache", "pa_copy_blocks",
    "pa_attention_workspace_size", "pa_attention_decode", "pa_attention_mixed",
    "pa_attention_decode_shared_prefix", "pa_attention_decode_shared_prefix_workspace_size",
    "pa_cache_and_attend_decode", "pa_cache_and_attend_mixed",
    "pa_cache_and_attend_decode_shared_prefix",
    "pa_cache_and_attend_mixed_no_workspace", "NO_WORKSPACE_MAX_BYTES",
    "pa_check_metadata", "META_FLAGS", "pa_status_string", "pa_version", "pa_read_probe",
    "pa_plan_decode_ranges",
    # short names: host bounds read back from the device when not given
    "compute_slot_mapping", "reshape_and_cache", "copy_blocks", "attention_decode",
    "attention_mixed", "cache_and_attend_decode", "cache_and_attend_mixed",
    "attention_decode_shared_prefix",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpa.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build the HIP library first "
        "(python paged_kv_attention_07_amd/build.py)")

# torch is imported before the library is loaded: libpa.so needs
# libamdhip64.so.7, and torch bundles its own copy under that soname.  Loading
# torch first makes the loader reuse torch's HIP runtime, so the device memory
# and streams torch hands over belong to the runtime that launches the
# kernels.  Loading libpa.so first would map a second HIP/HSA runtime into the
# process, and torch's allocations would be invalid for it.
import torch as _torch_module  # noqa: E402,F401

lib = ctypes.CDLL(library_path)

_i32, _i64, _sz, _f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                              ctypes.c_float, ctypes.c_void_p)

lib.pa_status_string.argtypes = [ctypes.c_int]
lib.pa_status_string.restype = ctypes.c_char_p
lib.pa_version.argtypes = []
lib.pa_version.restype = ctypes.c_int
lib.pa_compute_slot_mapping.argtypes = [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp]
lib.pa_compute_slot_mapping.restype = ctypes.c_int
lib.pa_reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp]
lib.pa_reshape_and_cache.restype = ctypes.c_int
lib.pa_copy_blocks.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp]
lib.pa_copy_blocks.restype = ctypes.c_int
lib.pa_attention_workspace_size.argtypes = [_i32] * 8
lib.pa_attention_workspace_size.restype = _sz
lib.pa_attention_decode.argtypes = [
    _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,   # out q kv NB B Hkv D dtype
    _vp, _i32, _vp, _i32, _i32, _i32, _f32,          # bt stride seq_lens R max_L Hq scale
    _vp, _sz, _i32, _vp]                             # ws ws_bytes splits stream
lib.pa_attention_decode.restype = ctypes.c_int
lib.pa_attention_mixed.argtypes = [
    _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,   # out q kv NB B Hkv D dtype
    _vp, _i32, _vp, _vp, _vp, _i32, _i32,            # bt stride seq_lens qsl nc R T
    _i32, _i32, _i32, _f32,                          # max_q max_L Hq scale
    _vp, _sz, _i32, _vp]                             # ws ws_bytes splits stream
lib.pa_attention_mixed.restype = ctypes.c_int
lib.pa_attention_decode_shared_prefix_workspace_size.argtypes = [_i32] * 7
lib.pa_attention_decode_shared_prefix_workspace_size.restype = _sz
lib.pa_attention_decode_shared_prefix.argtypes = [
    _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,   # out q kv NB B Hkv D dtype
    _vp, _i32, _vp, _i32, _i32, _i32, _f32,          # bt stride seq_lens R max_L Hq scale
    _i32, _vp, _sz, _i32, _vp]                       # prefix ws ws_bytes splits stream
lib.pa_attention_decode_shared_prefix.restype = ctypes.c_int

lib.pa_cache_and_attend_decode.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,  # out q key value kv NB B Hkv D dtype
    _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,              # bt stride seq_lens slots R max_L Hq scale
    _vp, _sz, _i32, _vp]                                      # ws ws_bytes splits stream
lib.pa_cache_and_attend_decode.restype = ctypes.c_int
lib.pa_cache_and_attend_decode_shared_prefix.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,  # out q key value kv NB B Hkv D dtype
    _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,              # bt stride seq_lens slots R max_L Hq scale
    _i32, _vp, _sz, _i32, _vp]                                # prefix ws ws_bytes splits stream
lib.pa_cache_and_attend_decode_shared_prefix.restype = ctypes.c_int
lib.pa_cache_and_attend_mixed.argtypes = [
    _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32,  # out q key value kv NB B Hkv D dtype
    _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32,                # bt stride seq_lens qsl nc slots R T
    _i32, _i32, _i32, _f32,                                   # max_q max_L Hq scale
    _vp, _sz, _i32, _vp]                                      # ws ws_bytes splits stream
lib.pa_cache_and_attend_mixed.restype = ctypes.c_int
lib.pa_cache_and_attend_mixed_no_workspace.argtypes = \
    lib.pa_cache_and_attend_mixed.argtypes[:-4] + [_i32, _vp]  # no ws, ws_bytes
lib.pa_cache_and_attend_mixed_no_workspace.restype = ctypes.c_int

# size of the library's built-in scratch array (PA_NO_WORKSPACE_MAX_BYTES)
NO_WORKSPACE_MAX_BYTES = 32 << 20

lib.pa_check_metadata.argtypes = [
    _vp, _vp, _i32, _vp, _vp, _vp, _vp,       # flags bt stride seq_lens qsl nc slots
    _i32, _i32, _i32, _i32, _i64, _i32, _i32,  # R T max_q max_L NB B prefix_blocks
    _vp]
lib.pa_check_metadata.restype = ctypes.c_int

class _MixedPlan(ctypes.Structure):
    _fields_ = [("num_splits", _i32), ("tile_shape", _i32), ("tiles_beside_decode", _i32)]


lib.pa_attention_mixed_planned.argtypes = lib.pa_attention_mixed.argtypes[:-2] + [
    ctypes.POINTER(_MixedPlan), _vp]
lib.pa_attention_mixed_planned.restype = ctypes.c_int
lib.pa_cache_and_attend_mixed_planned.argtypes = lib.pa_cache_and_attend_mixed.argtypes[:-2] + [
    ctypes.POINTER(_MixedPlan), _vp]
lib.pa_cache_and_attend_mixed_planned.restype = ctypes.c_int
lib.pa_plan_decode_ranges.argtypes = [_i32] * 9
lib.pa_plan_decode_ranges.restype = ctypes.c_int

lib.pa_read_probe.argtypes = [_vp, _sz, _vp, _i32, _vp]
lib.pa_read_probe.restype = ctypes.c_int

PA_F32, PA_BF16, PA_F16 = 0, 1, 2
DTYPE_CODES = {"f32": PA_F32, "bf16": PA_BF16, "f16": PA_F16}


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.pa_status_string(status).decode()} (status {status})")


def pa_status_string(status: int) -> str:
    return lib.pa_status_string(status).decode()


def pa_version() -> int:
    return lib.pa_version()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PAError(fn, status)


def _torch():
    return _torch_module


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.float16: PA_F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str, dtype=None, ndim: Optional[int] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _cache_dims(kv_cache):
    if kv_cache.dim() != 5 or kv_cache.shape[1] != 2:
        raise ValueError("kv_cache must be [num_blocks, 2, block_size, num_kv_heads, head_dim]")
    nb, _, bs, hkv, d = kv_cache.shape
    return int(nb), int(bs), int(hkv), int(d)


def pa_compute_slot_mapping(block_table, query_start_loc, num_computed_tokens,
                            num_tokens: int, block_size: int = 16, out=None):
    """Slot of every query token (int64 [num_tokens]); see pa.h."""
    torch = _torch()
    R = int(num_computed_tokens.shape[0])
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_table.device)
    st = lib.pa_compute_slot_mapping(
        _dev(out, "out", torch.int64, 1), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(query_start_loc, "query_start_loc", torch.int32, 1),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32, 1), R, int(num_tokens),
        int(block_size), _stream())
    _check("pa_compute_slot_mapping", st)
    return out


def pa_reshape_and_cache(key, value, kv_cache, slot_mapping) -> None:
    """Scatter key/value [T, Hkv, D] into kv_cache at slot_mapping [T] (int64)."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    T = int(key.shape[0])
    for name, t in (("key", key), ("value", value)):
        if tuple(t.shape) != (T, hkv, d) or t.dtype != kv_cache.dtype:
            raise ValueError(f"{name} must be [{T}, {hkv}, {d}] {kv_cache.dtype}")
    if tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    st = lib.pa_reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(kv_cache, "kv_cache"),
        _dev(slot_mapping, "slot_mapping", torch.int64, 1), T, nb, bs, hkv, d,
        _dtype_code(kv_cache), _stream())
    _check("pa_reshape_and_cache", st)


def pa_copy_blocks(kv_cache, block_pairs) -> None:
    """Copy whole cache blocks: kv_cache[dst] = kv_cache[src] for every
    (src, dst) row of block_pairs [P, 2] (int32, on the cache's device)."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    P = int(block_pairs.shape[0])
    st = lib.pa_copy_blocks(_dev(kv_cache, "kv_cache"),
                            _dev(block_pairs, "block_pairs", torch.int32, 2), P, nb, bs, hkv,
                            d, _dtype_code(kv_cache), _stream())
    _check("pa_copy_blocks", st)


def pa_attention_workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int,
                                num_kv_heads: int, head_dim: int, max_seq_len: int,
                                max_query_len: int, num_splits: int = 0) -> int:
    return int(lib.pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                               head_dim, max_seq_len, max_query_len, num_splits))


def _workspace(nbytes: int, device, workspace):
    """A caller-supplied workspace, or a new one (its contents on entry do not
    matter to the library; zero-filled here for reproducible debugging)."""
    torch = _torch()
    if workspace is None:
        return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace too small: need {nbytes} bytes")
    return workspace


def pa_attention_decode(q, kv_cache, block_table, seq_lens, scale: float, max_seq_len: int,
                        out=None, workspace=None, num_splits: int = 0):
    """One query token per request: q [R, Hq, D] -> out [R, Hq, D]; see pa.h."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    R, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(R, R, hq, hkv, d, max_seq_len, 1, num_splits)
    ws = _workspace(need, q.device, workspace)
    st = lib.pa_attention_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(kv_cache, "kv_cache"), nb, bs, hkv, d,
        _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1), R,
        int(max_seq_len), hq, float(scale), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), int(num_splits), _stream())
    _check("pa_attention_decode", st)
    return out


def pa_attention_decode_shared_prefix_workspace_size(num_seqs: int, num_q_heads: int,
                                                     num_kv_heads: int, head_dim: int,
                                                     max_seq_len: int, shared_prefix_blocks: int,
                                                     num_splits: int = 0) -> int:
    return lib.pa_attention_decode_shared_prefix_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, shared_prefix_blocks,
        num_splits)


def pa_attention_decode_shared_prefix(q, kv_cache, block_table, seq_lens, scale: float,
                                      max_seq_len: int, shared_prefix_blocks: int, out=None,
                                      workspace=None, num_splits: int = 0):
    """Decode where every request's first `shared_prefix_blocks` table entries
    are the same physical blocks: the prefix is read once; see pa.h."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    R, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_decode_shared_prefix_workspace_size(R, hq, hkv, d, max_seq_len,
                                                            shared_prefix_blocks, num_splits)
    if need == 0:
        raise ValueError("unsupported shared-prefix decode arguments")
    ws = _workspace(need, q.device, workspace)
    st = lib.pa_attention_decode_shared_prefix(
        _dev(out, "out"), _dev(q, "q"), _dev(kv_cache, "kv_cache"), nb, bs, hkv, d,
        _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1), R,
        int(max_seq_len), hq, float(scale), int(shared_prefix_blocks), _dev(ws, "workspace"),
        ws.numel() * ws.element_size(), int(num_splits), _stream())
    _check("pa_attention_decode_shared_prefix", st)
    return out


def _plan(num_splits, tile_shape, tiles_beside_decode):
    """A pa_mixed_plan, or None when the library chooses everything but the
    split count (the plain entry points)."""
    if tile_shape is None and tiles_beside_decode is None:
        return None
    return _MixedPlan(int(num_splits), -1 if tile_shape is None else int(tile_shape),
                      -1 if tiles_beside_decode is None else int(tiles_beside_decode))


def pa_attention_mixed(q, kv_cache, block_table, seq_lens, query_start_loc,
                       num_computed_tokens, scale: float, max_query_len: int,
                       max_seq_len: int, out=None, workspace=None, num_splits: int = 0,
                       tile_shape: Optional[int] = None,
                       tiles_beside_decode: Optional[int] = None):
    """Chunked-prefill mixed batch: q [T, Hq, D] varlen-packed -> out; see pa.h.
    ``tile_shape`` / ``tiles_beside_decode`` spell out the plan
    (pa_attention_mixed_planned); None leaves them to the library."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    T, hq = int(q.shape[0]), int(q.shape[1])
    R = int(seq_lens.shape[0])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_tokens, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(R, T, hq, hkv, d, max_seq_len, max_query_len, num_splits)
    ws = _workspace(need, q.device, workspace)
    args = (_dev(out, "out"), _dev(q, "q"), _dev(kv_cache, "kv_cache"), nb, bs, hkv, d,
            _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
            int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
            _dev(query_start_loc, "query_start_loc", torch.int32, 1),
            _dev(num_computed_tokens, "num_computed_tokens", torch.int32, 1), R, T,
            int(max_query_len), int(max_seq_len), hq, float(scale), _dev(ws, "workspace"),
            ws.numel() * ws.element_size())
    plan = _plan(num_splits, tile_shape, tiles_beside_decode)
    if plan is None:
        st = lib.pa_attention_mixed(*args, int(num_splits), _stream())
        _check("pa_attention_mixed", st)
    else:
        st = lib.pa_attention_mixed_planned(*args, ctypes.byref(plan), _stream())
        _check("pa_attention_mixed_planned", st)
    return out


def _new_rows(t, name, rows, hkv, d, kv_cache):
    if t.dim() != 3 or tuple(t.shape) != (rows, hkv, d) or t.dtype != kv_cache.dtype:
        raise ValueError(f"{name} must be [{rows}, num_kv_heads, head_dim] in the cache dtype")
    return _dev(t, name)


def _slots_out(slot_mapping, rows):
    torch = _torch()
    if slot_mapping is None:
        return None
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() < rows:
        raise ValueError("slot_mapping must be int64 with one entry per new token")
    return _dev(slot_mapping, "slot_mapping")


def pa_cache_and_attend_decode(q, key, value, kv_cache, block_table, seq_lens, scale: float,
                               max_seq_len: int, out=None, slot_mapping=None, workspace=None,
                               num_splits: int = 0):
    """Decode step in one launch: stores key/value [R, Hkv, D] at position
    seq_lens[r] - 1 of each request and attends; see pa.h."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    R, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(R, R, hq, hkv, d, max_seq_len, 1, num_splits)
    ws = _workspace(need, q.device, workspace)
    st = lib.pa_cache_and_attend_decode(
        _dev(out, "out"), _dev(q, "q"), _new_rows(key, "key", R, hkv, d, kv_cache),
        _new_rows(value, "value", R, hkv, d, kv_cache), _dev(kv_cache, "kv_cache"), nb, bs,
        hkv, d, _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
        _slots_out(slot_mapping, R), R, int(max_seq_len), hq, float(scale),
        _dev(ws, "workspace"), ws.numel() * ws.element_size(), int(num_splits), _stream())
    _check("pa_cache_and_attend_decode", st)
    return out


def pa_cache_and_attend_decode_shared_prefix(q, key, value, kv_cache, block_table, seq_lens,
                                             scale: float, max_seq_len: int,
                                             shared_prefix_blocks: int, out=None,
                                             slot_mapping=None, workspace=None,
                                             num_splits: int = 0):
    """Decode step of a batch sharing its first `shared_prefix_blocks` table
    entries, in one launch: stores key/value [R, Hkv, D] at position
    seq_lens[r] - 1 (past the prefix) and attends, the prefix read once; see
    pa.h."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    R, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_decode_shared_prefix_workspace_size(R, hq, hkv, d, max_seq_len,
                                                            shared_prefix_blocks, num_splits)
    if need == 0:
        raise ValueError("unsupported shared-prefix decode arguments")
    ws = _workspace(need, q.device, workspace)
    st = lib.pa_cache_and_attend_decode_shared_prefix(
        _dev(out, "out"), _dev(q, "q"), _new_rows(key, "key", R, hkv, d, kv_cache),
        _new_rows(value, "value", R, hkv, d, kv_cache), _dev(kv_cache, "kv_cache"), nb, bs,
        hkv, d, _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
        _slots_out(slot_mapping, R), R, int(max_seq_len), hq, float(scale),
        int(shared_prefix_blocks), _dev(ws, "workspace"), ws.numel() * ws.element_size(),
        int(num_splits), _stream())
    _check("pa_cache_and_attend_decode_shared_prefix", st)
    return out


def pa_cache_and_attend_mixed(q, key, value, kv_cache, block_table, seq_lens, query_start_loc,
                              num_computed_tokens, scale: float, max_query_len: int,
                              max_seq_len: int, out=None, slot_mapping=None, workspace=None,
                              num_splits: int = 0, tile_shape: Optional[int] = None,
                              tiles_beside_decode: Optional[int] = None):
    """Mixed step in one launch: stores key/value [T, Hkv, D] of every new
    token by its slot and attends; see pa.h.  The plan arguments as
    pa_attention_mixed."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    T, hq = int(q.shape[0]), int(q.shape[1])
    R = int(seq_lens.shape[0])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_tokens, num_q_heads, head_dim] in the cache dtype")
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(R, T, hq, hkv, d, max_seq_len, max_query_len, num_splits)
    ws = _workspace(need, q.device, workspace)
    args = (_dev(out, "out"), _dev(q, "q"), _new_rows(key, "key", T, hkv, d, kv_cache),
            _new_rows(value, "value", T, hkv, d, kv_cache), _dev(kv_cache, "kv_cache"), nb, bs,
            hkv, d, _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
            int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
            _dev(query_start_loc, "query_start_loc", torch.int32, 1),
            _dev(num_computed_tokens, "num_computed_tokens", torch.int32, 1),
            _slots_out(slot_mapping, T), R, T, int(max_query_len), int(max_seq_len), hq,
            float(scale), _dev(ws, "workspace"), ws.numel() * ws.element_size())
    plan = _plan(num_splits, tile_shape, tiles_beside_decode)
    if plan is None:
        st = lib.pa_cache_and_attend_mixed(*args, int(num_splits), _stream())
        _check("pa_cache_and_attend_mixed", st)
    else:
        st = lib.pa_cache_and_attend_mixed_planned(*args, ctypes.byref(plan), _stream())
        _check("pa_cache_and_attend_mixed_planned", st)
    return out


def pa_plan_decode_ranges(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          dtype: str, max_seq_len: int, max_query_len: int = 1,
                          num_splits: int = 0, num_cus: int = 256) -> int:
    """Key ranges per KV head the split plans on a device of `num_cus`
    compute units (a pure query; see pa.h)."""
    st = lib.pa_plan_decode_ranges(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                   DTYPE_CODES[dtype], max_seq_len, max_query_len, num_splits,
                                   num_cus)
    if st < 0:
        raise PAError("pa_plan_decode_ranges", st)
    return st


def pa_cache_and_attend_mixed_no_workspace(q, key, value, kv_cache, block_table, seq_lens,
                                           query_start_loc, num_computed_tokens, scale: float,
                                           max_query_len: int, max_seq_len: int, out,
                                           slot_mapping=None, num_splits: int = 0):
    """pa_cache_and_attend_mixed with the split partials in the library's own
    scratch array: allocates nothing, so ``out`` must be given; see pa.h."""
    torch = _torch()
    nb, bs, hkv, d = _cache_dims(kv_cache)
    T, hq = int(q.shape[0]), int(q.shape[1])
    R = int(seq_lens.shape[0])
    if q.dim() != 3 or int(q.shape[2]) != d or q.dtype != kv_cache.dtype:
        raise ValueError("q must be [num_tokens, num_q_heads, head_dim] in the cache dtype")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must have q's shape and dtype")
    st = lib.pa_cache_and_attend_mixed_no_workspace(
        _dev(out, "out"), _dev(q, "q"), _new_rows(key, "key", T, hkv, d, kv_cache),
        _new_rows(value, "value", T, hkv, d, kv_cache), _dev(kv_cache, "kv_cache"), nb, bs,
        hkv, d, _dtype_code(kv_cache), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(query_start_loc, "query_start_loc", torch.int32, 1),
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32, 1),
        _slots_out(slot_mapping, T), R, T, int(max_query_len), int(max_seq_len), hq,
        float(scale), int(num_splits), _stream())
    _check("pa_cache_and_attend_mixed_no_workspace", st)
    return out


def pa_read_probe(buf, sink, waves_per_simd: int = 1) -> None:
    """Stream the bytes of GPU tensor `buf` through the load units (the
    read-bandwidth reference of include/pa_probe.h); `sink` is a one-element
    int32 GPU tensor the kernel may write."""
    torch = _torch()
    st = lib.pa_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                           _dev(sink, "sink", torch.int32, 1), int(waves_per_simd), _stream())
    _check("pa_read_probe", st)


# pa_meta_flag bits of pa_check_metadata (include/pa.h), in bit order
META_FLAGS = ("seq_len", "table_width", "block_id", "query_start", "computed", "query_len",
              "slot_range", "slot_dup", "shared_prefix")


def pa_check_metadata(block_table, seq_lens, num_blocks: int, max_seq_len: int,
                      query_start_loc=None, num_computed_tokens=None, slot_mapping=None,
                      num_tokens: Optional[int] = None, max_query_len: Optional[int] = None,
                      shared_prefix_blocks: int = 0, block_size: int = 16, flags=None):
    """Check the step metadata on the device; see pa.h.  ``num_tokens`` is the
    caller's token count for a mixed batch (default: the slot_mapping length,
    else query_start_loc[-1], read back).  With ``flags`` (a zeroed one-element
    int32 GPU tensor) the call only launches and returns ``flags``; without,
    it synchronises the stream and returns the names of the violated
    conditions (empty: all hold)."""
    torch = _torch()
    R = int(seq_lens.shape[0])
    mixed = query_start_loc is not None
    if mixed and (num_computed_tokens is None or int(query_start_loc.shape[0]) != R + 1):
        raise ValueError("a mixed batch needs query_start_loc [R+1] and num_computed_tokens [R]")
    if not mixed:
        T = R
    elif num_tokens is not None:
        T = int(num_tokens)
    elif slot_mapping is not None:
        T = int(slot_mapping.shape[0])
    else:
        T = int(query_start_loc[-1].item())
    if slot_mapping is not None and int(slot_mapping.shape[0]) != T:
        raise ValueError(f"slot_mapping must have {T} entries")
    if max_query_len is None:
        max_query_len = 1 if not mixed else T
    own = flags is None
    if own:
        flags = torch.zeros(1, dtype=torch.int32, device=seq_lens.device)
    st = lib.pa_check_metadata(
        _dev(flags, "flags", torch.int32, 1), _dev(block_table, "block_table", torch.int32, 2),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32, 1),
        _dev(query_start_loc, "query_start_loc", torch.int32, 1) if mixed else None,
        _dev(num_computed_tokens, "num_computed_tokens", torch.int32, 1) if mixed else None,
        _dev(slot_mapping, "slot_mapping", torch.int64, 1) if slot_mapping is not None else None,
        R, T, int(max_query_len), int(max_seq_len), int(num_blocks), int(block_size),
        int(shared_prefix_blocks), _stream())
    _check("pa_check_metadata", st)
    if not own:
        return flags
    torch.cuda.current_stream().synchronize()
    bits = int(flags.item()) & 0xFFFFFFFF
    return [name for i, name in enumerate(META_FLAGS) if bits >> i & 1]


# ---- short names ------------------------------------------------------------
# The pa_* functions take the host bounds (max_seq_len, max_query_len) as
# arguments, as the C ABI does, so they never synchronise.  These short forms
# follow the pages' call shapes; a bound left as None is read back from the
# device metadata (one synchronisation of the current stream).


def _max_of(t) -> int:
    return int(t.max().item()) if t.numel() else 0


def _max_query_len(query_start_loc) -> int:
    return _max_of(query_start_loc[1:] - query_start_loc[:-1]) if query_start_loc.numel() > 1 else 0


compute_slot_mapping = pa_compute_slot_mapping
reshape_and_cache = pa_reshape_and_cache
copy_blocks = pa_copy_blocks


def attention_decode(q, kv_cache, block_table, seq_lens, scale: float,
                     max_seq_len: Optional[int] = None, **kw):
    """pa_attention_decode with max_seq_len defaulting to max(seq_lens)."""
    if max_seq_len is None:
        max_seq_len = _max_of(seq_lens)
    return pa_attention_decode(q, kv_cache, block_table, seq_lens, scale, max_seq_len, **kw)


def attention_decode_shared_prefix(q, kv_cache, block_table, seq_lens, scale: float,
                                   shared_prefix_blocks: int, max_seq_len: Optional[int] = None,
                                   **kw):
    if max_seq_len is None:
        max_seq_len = _max_of(seq_lens)
    return pa_attention_decode_shared_prefix(q, kv_cache, block_table, seq_lens, scale,
                                             max_seq_len, shared_prefix_blocks, **kw)


def attention_mixed(q, kv_cache, block_table, seq_lens, query_start_loc, num_computed_tokens,
                    scale: float, max_query_len: Optional[int] = None,
                    max_seq_len: Optional[int] = None, **kw):
    """pa_attention_mixed with the bounds defaulting to the batch's own."""
    if max_query_len is None:
        max_query_len = _max_query_len(query_start_loc)
    if max_seq_len is None:
        max_seq_len = _max_of(seq_lens)
    return pa_attention_mixed(q, kv_cache, block_table, seq_lens, query_start_loc,
                              num_computed_tokens, scale, max_query_len, max_seq_len, **kw)


def cache_and_attend_decode(q, key, value, kv_cache, block_table, seq_lens, scale: float,
                            max_seq_len: Optional[int] = None, **kw):
    if max_seq_len is None:
        max_seq_len = _max_of(seq_lens)
    return pa_cache_and_attend_decode(q, key, value, kv_cache, block_table, seq_lens, scale,
                                      max_seq_len, **kw)


def cache_and_attend_mixed(q, key, value, kv_cache, block_table, seq_lens, query_start_loc,
                           num_computed_tokens, scale: float, max_query_len: Optional[int] = None,
                           max_seq_len: Optional[int] = None, **kw):
    if max_query_len is None:
        max_query_len = _max_query_len(query_start_loc)
    if max_seq_len is None:
        max_seq_len = _max_of(seq_lens)
    return pa_cache_and_attend_mixed(q, key, value, kv_cache, block_table, seq_lens,
                                     query_start_loc, num_computed_tokens, scale, max_query_len,
                                     max_seq_len, **kw)
