"""Helpers for the GPU parity tests: move seeded workloads to the device, run
the HIP path through the C ABI, and run the oracle on the same host bits."""

from __future__ import annotations

import numpy as np

import oracle

# tolerances against the fp64 oracle
TOL = {
    "f32": dict(max_abs=1e-5, mean_abs=1e-5),
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3),
    "f16": dict(max_abs=2e-2, mean_abs=2e-3),
}


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch_dtype(dtype))
    return t.to("cuda")


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().to("cpu").contiguous()
    if dtype == "f32":
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def ints_to_device(a: np.ndarray, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to("cuda")


def bits(a: np.ndarray) -> np.ndarray:
    """Integer view for bit-exact comparison (NaN payloads included)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def poisoned_pool(w) -> np.ndarray:
    """The pool with NaN in every slot attention must not read before the
    step's scatter: slots outside each request's 0..seq_len-1 positions and
    the slots this step's tokens are about to be written to."""
    pool = w.pool.copy()
    used = oracle.used_slot_mask(w.block_table, w.seq_lens, w.num_blocks, w.block_size)
    slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size)
    used[slots // w.block_size, slots % w.block_size] = False
    nan = np.float32(np.nan) if w.dtype == "f32" else (
        np.uint16(0x7FC0) if w.dtype == "bf16" else np.uint16(0x7E00))
    blk, off = np.nonzero(~used)
    pool[blk, :, off] = nan
    return pool


class Device:
    """A workload's tensors on the GPU."""

    def __init__(self, w, pool: np.ndarray = None):
        self.w = w
        self.kv = to_device(w.pool if pool is None else pool, w.dtype)
        self.q = to_device(w.q, w.dtype)
        self.k_new = to_device(w.k_new, w.dtype)
        self.v_new = to_device(w.v_new, w.dtype)
        self.block_table = ints_to_device(w.block_table, np.int32)
        self.seq_lens = ints_to_device(w.seq_lens, np.int32)
        self.qsl = ints_to_device(w.query_start_loc, np.int32)
        self.num_computed = ints_to_device(w.num_computed, np.int32)

    def slot_mapping(self):
        import paged_kv_attention_07_amd as pa
        return pa.pa_compute_slot_mapping(self.block_table, self.qsl, self.num_computed,
                                          self.w.num_tokens, self.w.block_size)

    def scatter(self, slots):
        import paged_kv_attention_07_amd as pa
        pa.pa_reshape_and_cache(self.k_new, self.v_new, self.kv, slots)

    def attend(self, num_splits=0, force_mixed=False, shared_prefix=None, plan=None):
        """`plan`: keyword arguments spelling out a mixed batch's plan
        (tile_shape, tiles_beside_decode) for pa_attention_mixed."""
        import paged_kv_attention_07_amd as pa
        w = self.w
        if shared_prefix is not None:
            return pa.pa_attention_decode_shared_prefix(
                self.q, self.kv, self.block_table, self.seq_lens, w.scale, w.max_seq_len,
                shared_prefix, num_splits=num_splits)
        if w.is_decode_only and not force_mixed:
            return pa.pa_attention_decode(self.q, self.kv, self.block_table, self.seq_lens,
                                          w.scale, w.max_seq_len, num_splits=num_splits)
        return pa.pa_attention_mixed(self.q, self.kv, self.block_table, self.seq_lens, self.qsl,
                                     self.num_computed, w.scale, w.max_query_len, w.max_seq_len,
                                     num_splits=num_splits, **(plan or {}))


    def cache_and_attend(self, num_splits=0, force_mixed=False, slots=True,
                         shared_prefix=None, plan=None):
        """The one-launch step: the attention call stores the new tokens
        itself.  Returns (out, slot_mapping or None); the slot buffer starts
        at -7 so an entry the library does not write shows."""
        import torch
        import paged_kv_attention_07_amd as pa
        w = self.w
        sm = (torch.full((w.num_tokens,), -7, dtype=torch.int64, device="cuda")
              if slots else None)
        if shared_prefix is not None:
            out = pa.pa_cache_and_attend_decode_shared_prefix(
                self.q, self.k_new, self.v_new, self.kv, self.block_table, self.seq_lens,
                w.scale, w.max_seq_len, shared_prefix, slot_mapping=sm, num_splits=num_splits)
        elif w.is_decode_only and not force_mixed:
            out = pa.pa_cache_and_attend_decode(self.q, self.k_new, self.v_new, self.kv,
                                                self.block_table, self.seq_lens, w.scale,
                                                w.max_seq_len, slot_mapping=sm,
                                                num_splits=num_splits)
        else:
            out = pa.pa_cache_and_attend_mixed(self.q, self.k_new, self.v_new, self.kv,
                                               self.block_table, self.seq_lens, self.qsl,
                                               self.num_computed, w.scale, w.max_query_len,
                                               w.max_seq_len, slot_mapping=sm,
                                               num_splits=num_splits, **(plan or {}))
        return out, sm


def run_step(w, *, poison=True, num_splits=0, force_mixed=False, shared_prefix=None,
             fused=False, plan=None):
    """Slot mapping, scatter and attention on the GPU for one step of `w`
    (fused: one cache-and-attend call).  Returns (pool_before, gpu_slots,
    gpu_pool, gpu_out) as host arrays."""
    import torch
    pool = poisoned_pool(w) if poison else w.pool
    dev = Device(w, pool)
    if fused:
        out, slots = dev.cache_and_attend(num_splits=num_splits, force_mixed=force_mixed,
                                          shared_prefix=shared_prefix, plan=plan)
    else:
        slots = dev.slot_mapping()
        dev.scatter(slots)
        out = dev.attend(num_splits=num_splits, force_mixed=force_mixed,
                         shared_prefix=shared_prefix, plan=plan)
    torch.cuda.synchronize()
    return pool, slots.cpu().numpy(), from_device(dev.kv, w.dtype), from_device(out, w.dtype)


def oracle_step(w, pool, requests=None):
    slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size)
    pool_after = oracle.reshape_and_cache(pool, w.k_new, w.v_new, slots)
    out = oracle.paged_attention(w.q, pool_after, w.block_table, w.seq_lens, w.query_start_loc,
                                 w.num_computed, w.scale, w.dtype, requests=requests)
    return slots, pool_after, out


def rows_of(w, requests):
    qsl = w.query_start_loc
    return np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in requests]).astype(np.int64)


def check_close(w, got_bits: np.ndarray, want: np.ndarray, rows=None, what=""):
    got = oracle.decode_bits(got_bits, w.dtype)
    if rows is not None:
        got, want = got[rows], want[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    tol = TOL[w.dtype]
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= tol["max_abs"], f"{what}: max abs err {mx:.3g} > {tol['max_abs']}"
    assert mean <= tol["mean_abs"], f"{what}: mean abs err {mean:.3g} > {tol['mean_abs']}"
    return mx, mean


def sampled_rows_check(w, dev_out_bits, rows):
    """Compare selected query rows with the oracle, each row computed as its
    own one-token request at its absolute position (same table, same pool)."""
    import dataclasses
    qsl = w.query_start_loc
    req_of = np.searchsorted(qsl, np.asarray(rows), side="right") - 1
    nc = np.array([w.num_computed[r] + (t - qsl[r]) for t, r in zip(rows, req_of)], np.int32)
    sub = dataclasses.replace(
        w, q=w.q[rows], seq_lens=(nc + 1).astype(np.int32), num_computed=nc,
        query_start_loc=np.arange(len(rows) + 1, dtype=np.int32),
        block_table=w.block_table[req_of])
    return sub
