"""The one-launch steps inside a captured HIP graph (torch.cuda.CUDAGraph):
serving loops capture a decode step once and replay it.  The entry points
launch kernels only (no allocation, no memset, no host synchronisation), so a
capture must replay to the eager result bit for bit, every time, with other
eager work on the device between replays.
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


def _buffers(w, dev):
    need = pa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads,
                                          w.num_kv_heads, w.head_dim, w.max_seq_len,
                                          w.max_query_len, 0)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev.q)
    slots = torch.full((w.num_tokens,), -7, dtype=torch.int64, device="cuda")
    return ws, out, slots


def _step(w, dev, ws, out, slots):
    if w.is_decode_only:
        pa.pa_cache_and_attend_decode(dev.q, dev.k_new, dev.v_new, dev.kv, dev.block_table,
                                      dev.seq_lens, w.scale, w.max_seq_len, out=out,
                                      slot_mapping=slots, workspace=ws)
    else:
        pa.pa_cache_and_attend_mixed(dev.q, dev.k_new, dev.v_new, dev.kv, dev.block_table,
                                     dev.seq_lens, dev.qsl, dev.num_computed, w.scale,
                                     w.max_query_len, w.max_seq_len, out=out,
                                     slot_mapping=slots, workspace=ws)


@pytest.mark.parametrize("name", ["decode_bf16_small", "mixed_bf16_small", "long_decode_small"])
def test_step_replays_from_a_graph(name):
    w = make_workload(name)
    print(f"[case] graph {name}", flush=True)
    dev = gu.Device(w, gu.poisoned_pool(w))
    ws, out, slots = _buffers(w, dev)
    # eager reference (the cache holds the new tokens afterwards; a replay
    # stores the same bits again)
    _step(w, dev, ws, out, slots)
    torch.cuda.synchronize()
    ref_out = gu.from_device(out, w.dtype).copy()
    ref_pool = gu.from_device(dev.kv, w.dtype).copy()
    ref_slots = slots.cpu().numpy().copy()
    _, _, r_out = gu.oracle_step(w, gu.poisoned_pool(w))
    gu.check_close(w, ref_out, r_out, what=f"{name} eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(w, dev, ws, out, slots)        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, dev, ws, out, slots)
    scratch = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    for rep in range(4):
        out.zero_()
        slots.fill_(-7)
        ws.fill_(0xAB)                       # the workspace's contents must not matter
        scratch.normal_()                    # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.bits(gu.from_device(out, w.dtype)), gu.bits(ref_out)), rep
        assert np.array_equal(gu.bits(gu.from_device(dev.kv, w.dtype)), gu.bits(ref_pool)), rep
        assert np.array_equal(slots.cpu().numpy(), ref_slots), rep
