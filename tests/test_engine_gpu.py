"""End to end on the GPU: the C++ scheduler driving the HIP kernels over a
seeded multi-step trace (prefix hits, chunked prefill, preemption,
copy-on-write forks), checked every step against the oracle scheduler plus
the fp64 oracle over its own copy of the cache."""

import numpy as np
import pytest

import gpu_util as gu
import oracle
from oracle import sched as S
from workloads.trace import step_inputs, trace

pytestmark = pytest.mark.gpu

pa = pytest.importorskip("paged_kv_attention_07_amd")


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 8, 2, 128), ("f16", 4, 4, 64),
                                            ("f32", 16, 2, 128)])
def test_engine_matches_oracle_every_step(dtype, Hq, Hkv, D):
    import torch
    from paged_kv_attention_07_amd.engine import Engine
    t = trace("engine_small")
    B = t.block_size
    eng = Engine(num_blocks=t.num_blocks, max_num_batched_tokens=t.max_num_batched_tokens,
                 max_num_seqs=t.max_num_seqs, max_model_len=t.max_model_len, num_q_heads=Hq,
                 num_kv_heads=Hkv, head_dim=D, dtype=dtype)
    o = S.Scheduler(t.num_blocks, B, t.max_num_batched_tokens, t.max_num_seqs, t.max_model_len)
    if dtype == "f32":
        pool = np.full((t.num_blocks, 2, B, Hkv, D), np.nan, np.float32)
    else:
        nan = np.uint16(0x7FC0) if dtype == "bf16" else np.uint16(0x7E00)
        pool = np.full((t.num_blocks, 2, B, Hkv, D), nan, np.uint16)
    width = -(-t.max_model_len // B)
    seen = {"copies": 0, "preempted": 0, "prefill_rows": 0, "steps": 0}
    for step in range(t.num_steps):
        for rid, prompt, n in t.arrivals.get(step, []):
            eng.add_request(rid, prompt, n)
            o.add_request(rid, prompt, n)
        for parent, child, n in t.forks.get(step, []):
            assert eng.fork(parent, child, n) == o.fork(parent, child, n)
        ro = o.schedule()
        T = ro.num_tokens
        q, k, v = step_inputs(t.seed, step, max(T, 1), Hq, Hkv, D, dtype)
        qd, kd, vd = (gu.to_device(x, dtype) for x in (q, k, v))
        print(f"[engine] {dtype} step {step}: {len(ro.request_ids)} seqs, {T} tokens", flush=True)
        st = eng.step(qd, kd, vd)
        assert st.request_ids.tolist() == ro.request_ids
        assert st.num_new.tolist() == ro.num_new
        if T:
            got = gu.from_device(eng.out[:T], dtype)
            torch.cuda.synchronize()
            # oracle side: its own cache, its own metadata
            pool = oracle.copy_blocks(pool, np.array(ro.copies, np.int64).reshape(-1, 2))
            bt = np.full((len(ro.request_ids), width), -1, np.int32)
            for i, tab in enumerate(ro.block_tables):
                bt[i, :len(tab)] = tab
            qsl = np.concatenate([[0], np.cumsum(ro.num_new)]).astype(np.int32)
            nc = np.array(ro.num_computed, np.int32)
            slots = oracle.slot_mapping(bt, qsl, nc, B)
            pool = oracle.reshape_and_cache(pool, k[:T], v[:T], slots)
            ref = oracle.paged_attention(q[:T], pool, bt, nc + np.array(ro.num_new, np.int32),
                                         qsl, nc, eng.scale, dtype)
            w = type("W", (), {"dtype": dtype})
            gu.check_close(w, got, ref, what=f"step {step}")
            seen["copies"] += len(ro.copies)
            seen["preempted"] += len(ro.preempted)
            seen["prefill_rows"] += int(sum(n for n in ro.num_new if n > 1))
            seen["steps"] += 1
        sampled = [t.sampled(r, o.requests[r].num_generated) for r in ro.request_ids]
        assert eng.update(sampled) == o.update(sampled)
    assert all(r.status == S.FINISHED for r in o.requests.values())
    assert seen["copies"] and seen["preempted"] and seen["prefill_rows"]
    assert o.total_prefix_hit_tokens > 0
    # the GPU cache holds exactly the oracle's bits wherever the oracle wrote
    g_pool = gu.from_device(eng.kv, dtype)
    written = ~np.isnan(oracle.decode_bits(pool, dtype))
    assert np.array_equal(gu.bits(g_pool[written]), gu.bits(pool[written]))


def test_engine_runs_the_serving_trace():
    """The serving trace (256 requests, prompts of 64-1536 tokens, shared system
    prompts, chunked prefill under a 2048-token budget) through the native
    engine: every step's attention call succeeds with the engine's one
    workspace, sized once for the largest plan any step can need (steps mix
    short and long chunks with decode rows), and the schedule matches the
    oracle scheduler's step for step."""
    import torch
    from paged_kv_attention_07_amd.engine import Engine
    t = trace("serve_llama3_2k")
    Hq, Hkv, D = 32, 8, 128
    q, k, v = step_inputs(t.seed, 0, t.max_num_batched_tokens, Hq, Hkv, D, "bf16")
    qd, kd, vd = (gu.to_device(x, "bf16") for x in (q, k, v))
    eng = Engine(num_blocks=t.num_blocks, max_num_batched_tokens=t.max_num_batched_tokens,
                 max_num_seqs=t.max_num_seqs, max_model_len=t.max_model_len, num_q_heads=Hq,
                 num_kv_heads=Hkv, head_dim=D, dtype="bf16")
    o = S.Scheduler(t.num_blocks, t.block_size, t.max_num_batched_tokens, t.max_num_seqs,
                    t.max_model_len)
    tokens = chunk_steps = 0
    for step in range(t.num_steps):
        for rid, prompt, n in t.arrivals.get(step, []):
            eng.add_request(rid, prompt, n)
            o.add_request(rid, prompt, n)
        for parent, child, n in t.forks.get(step, []):
            assert eng.fork(parent, child, n) == o.fork(parent, child, n)
        ro = o.schedule()
        st = eng.step(qd, kd, vd)                      # raises on any non-zero status
        assert st.request_ids.tolist() == ro.request_ids, step
        assert st.num_new.tolist() == ro.num_new, step
        tokens += st.num_tokens
        chunk_steps += int(any(n > 1 for n in ro.num_new) and any(n == 1 for n in ro.num_new))
        sampled = [t.sampled(r, o.requests[r].num_generated) for r in ro.request_ids]
        assert eng.update(sampled) == o.update(sampled)
    torch.cuda.synchronize()
    assert torch.isfinite(eng.out.float()).all()
    assert all(r.status == S.FINISHED for r in o.requests.values())
    assert tokens > 100000 and chunk_steps > 10
    print(f"[engine] serving trace: {tokens} tokens, {chunk_steps} steps mixing chunks and "
          f"decode rows", flush=True)
