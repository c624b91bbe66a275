"""Calls on several streams at once.

The entry points keep no state between calls and touch only the buffers they
are given (each call its own workspace), so steps of different batches issued
on different streams, with no synchronisation between them, must give the
same bits as the same steps run one after the other on one stream.  Four
batches of different shapes (decode, mixed, long-context decode, shared
prefix) each run 5 one-launch steps on their own stream, interleaved call by
call; every output, slot list and pool is compared with a sequential run.
Streams are created at the default priority.
"""

import numpy as np
import pytest

from workloads import make_workload

import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_07_amd as pa  # noqa: E402  (fails loudly if libpa.so is missing)

NAMES = ["decode_bf16_small", "mixed_bf16_small", "long_decode_small", "prefix_shared_small"]
STEPS = 5


class Batch:
    def __init__(self, name):
        self.w = make_workload(name)
        self.prefix = int(self.w.meta.get("shared_prefix_blocks", 0))
        self.reset()

    def reset(self):
        w = self.w
        self.dev = gu.Device(w, gu.poisoned_pool(w))
        need = max(pa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads,
                                                  w.num_kv_heads, w.head_dim, w.max_seq_len,
                                                  w.max_query_len, 0),
                   pa.pa_attention_decode_shared_prefix_workspace_size(
                       w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_seq_len,
                       self.prefix) if self.prefix else 0)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        self.outs = [torch.empty_like(self.dev.q) for _ in range(STEPS)]
        self.slots = [torch.full((w.num_tokens,), -7, dtype=torch.int64, device="cuda")
                      for _ in range(STEPS)]

    def step(self, i):
        w, d = self.w, self.dev
        if self.prefix:
            pa.pa_cache_and_attend_decode_shared_prefix(
                d.q, d.k_new, d.v_new, d.kv, d.block_table, d.seq_lens, w.scale, w.max_seq_len,
                self.prefix, out=self.outs[i], slot_mapping=self.slots[i], workspace=self.ws)
        elif w.is_decode_only:
            pa.pa_cache_and_attend_decode(d.q, d.k_new, d.v_new, d.kv, d.block_table, d.seq_lens,
                                          w.scale, w.max_seq_len, out=self.outs[i],
                                          slot_mapping=self.slots[i], workspace=self.ws)
        else:
            pa.pa_cache_and_attend_mixed(d.q, d.k_new, d.v_new, d.kv, d.block_table, d.seq_lens,
                                         d.qsl, d.num_computed, w.scale, w.max_query_len,
                                         w.max_seq_len, out=self.outs[i],
                                         slot_mapping=self.slots[i], workspace=self.ws)

    def result(self):
        dt = self.w.dtype
        return ([gu.from_device(o, dt).copy() for o in self.outs],
                [s.cpu().numpy().copy() for s in self.slots], gu.from_device(self.dev.kv, dt).copy())


def test_concurrent_streams_match_sequential():
    batches = [Batch(n) for n in NAMES]
    print("[case] streams: sequential reference", flush=True)
    for b in batches:
        for i in range(STEPS):
            b.step(i)
    torch.cuda.synchronize()
    want = [b.result() for b in batches]
    for b in batches:
        b.reset()
    torch.cuda.synchronize()
    print("[case] streams: interleaved on 4 streams", flush=True)
    streams = [torch.cuda.Stream() for _ in batches]
    for i in range(STEPS):
        for b, s in zip(batches, streams):
            with torch.cuda.stream(s):
                b.step(i)
    torch.cuda.synchronize()
    for name, b, (w_outs, w_slots, w_pool) in zip(NAMES, batches, want):
        outs, slots, pool = b.result()
        for i in range(STEPS):
            assert np.array_equal(gu.bits(outs[i]), gu.bits(w_outs[i])), f"{name} step {i} output"
            assert np.array_equal(slots[i], w_slots[i]), f"{name} step {i} slots"
        assert np.array_equal(gu.bits(pool), gu.bits(w_pool)), f"{name} pool"
    # and the first step of each batch is right (the later ones store the same rows again)
    for name, (w_outs, _, _) in zip(NAMES, want):
        w = make_workload(name)
        _, _, r_out = gu.oracle_step(w, gu.poisoned_pool(w))
        gu.check_close(w, w_outs[0], r_out, what=f"{name} step 0")
