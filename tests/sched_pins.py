"""Checks that pin the scheduler / block-manager oracle to the pages' worked
examples and to invariants (called by test_sched_oracle.py; the mutation
test plants mistakes in the oracle and requires one of them to fail).
Sources are cited by page title and section:
  [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成"
  [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
  [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"
"""

from __future__ import annotations

import numpy as np

from oracle import sched as S

B = 16


def _step(s, sampled_base=0):
    out = s.schedule()
    s.update([sampled_base + i for i in range(len(out.request_ids))])
    s.check_invariants()
    return out


def check_chunk_sizes_worked_example():
    """[P4] §4.2: budget 256, two decodes running, a 1000-token prompt is
    prefilled in chunks of 254, 254, 254, 238, mixed with the decodes."""
    s = S.Scheduler(num_blocks=200, block_size=B, max_num_batched_tokens=256, max_num_seqs=8,
                    max_model_len=2048)
    s.add_request(0, list(range(10)), 100)
    s.add_request(1, list(range(20, 30)), 100)
    _step(s)                                  # both prompts in one step
    s.add_request(2, list(range(1000, 2000)), 4)
    chunks = []
    for _ in range(4):
        out = _step(s)
        assert out.request_ids[:2] == [0, 1] and out.num_new[:2] == [1, 1]
        chunks.append(out.num_new[2])
        assert out.num_tokens <= 256
    assert chunks == [254, 254, 254, 238]
    assert s.requests[2].num_generated == 1   # sampled only after the last chunk


def check_threshold_chunks():
    """[P1] §3.2 / [P2] §3.5: long_prefill_token_threshold caps a chunk."""
    s = S.Scheduler(200, B, 256, 8, 2048, long_prefill_token_threshold=100)
    s.add_request(0, list(range(250)), 2)
    assert [_step(s).num_new[0] for _ in range(3)] == [100, 100, 50]


def check_allocate_slots_block_count():
    """[P2] §3.3: 17 new tokens need ceil(17/16) = 2 blocks."""
    s = S.Scheduler(10, B, 256, 8, 512)
    s.add_request(0, list(range(17)), 1)
    out = s.schedule()
    assert len(out.block_tables[0]) == 2 and s.pool.num_free() == 8


def check_new_block_on_len_mod_1():
    """[P1] §4.3.3 (blocks allocated on demand while decoding): a decode step
    takes a new block exactly when the token it writes starts a block, i.e.
    when the sequence length becomes 1 mod 16."""
    s = S.Scheduler(40, B, 64, 4, 512)
    s.add_request(0, list(range(5)), 120)
    _step(s)
    r = s.requests[0]
    while r.status == S.RUNNING:
        before = len(r.blocks)
        out = s.schedule()
        L = out.num_computed[0] + out.num_new[0]          # length after the write
        assert (len(r.blocks) - before == 1) == (L % B == 1)
        assert len(r.blocks) == -(-L // B)
        s.update([7])


def check_prefix_hit_sets_computed():
    """[P4] §3.5: a hit on the first 2 blocks sets num_computed to 32 and only
    the rest is prefilled; the hit stops at the first differing block."""
    s = S.Scheduler(50, B, 256, 8, 512)
    base = list(range(100, 148))                          # 3 full blocks
    s.add_request(0, base, 20)
    _step(s)
    other = base[:32] + [1, 2, 3] + list(range(500, 513))  # block 2 differs
    s.add_request(1, other, 2)
    out = _step(s)
    i = out.request_ids.index(1)
    assert out.num_computed[i] == 32 and out.num_new[i] == len(other) - 32
    assert out.block_tables[i][:2] == s.requests[0].blocks[:2]
    assert out.block_tables[i][2] != s.requests[0].blocks[2]
    # a later block matching is no hit once an earlier one missed
    third = base[:16] + [9] * 16 + base[32:48] + [4]
    s.add_request(2, third, 1)
    out = _step(s)
    i = out.request_ids.index(2)
    assert out.num_computed[i] == 16
    # a prompt that is cached whole still computes its last block
    s.add_request(3, base, 1)
    out = _step(s)
    i = out.request_ids.index(3)
    assert out.num_computed[i] == 32 and out.num_new[i] == 16


def check_shared_system_prompt_refcounts():
    """[P1] §4.3.1: three requests with the same 100-token system prompt share
    its 6 full blocks (ref count 3); releasing one request drops the counts to
    2 and frees none of them."""
    s = S.Scheduler(60, B, 512, 8, 512)
    system = list(range(3000, 3100))
    s.add_request(1, system + [1, 2], 50)
    _step(s)
    s.add_request(2, system + [5, 6, 7], 50)
    s.add_request(3, system + [8, 9, 10, 11], 50)
    _step(s)
    t1, t2, t3 = (s.requests[i].blocks for i in (1, 2, 3))
    assert t1[:6] == t2[:6] == t3[:6]
    assert len({t1[6], t2[6], t3[6]}) == 3
    assert all(s.pool.blocks[b].ref_cnt == 3 for b in t1[:6])
    s.requests[1].max_new_tokens = s.requests[1].num_generated + 1
    _step(s)
    assert s.requests[1].status == S.FINISHED
    assert all(s.pool.blocks[b].ref_cnt == 2 for b in t2[:6])
    assert not set(t2[:6]) & set(s.pool.free)


def check_free_queue_order_and_reuse():
    """[P4] §3.3 / §3.6: freed blocks without a hash go to the head of the
    free queue (reused first), hashed ones to the tail; a finished request's
    hashed blocks still serve prefix hits ([P2] §3.6) until reallocated."""
    s = S.Scheduler(12, B, 256, 4, 512)
    prompt = list(range(40))                              # 2 full blocks + 8 tokens
    s.add_request(0, prompt, 1)
    out = _step(s)                                        # prefill, sample, finish
    b0, b1, b2 = out.block_tables[0]
    assert s.requests[0].status == S.FINISHED
    assert s.pool.free[0] == b2 and s.pool.blocks[b2].hash is None
    assert s.pool.free[-2:] == [b1, b0]                   # last block released first
    s.add_request(1, prompt[:32] + [77] * 8, 1)
    out = _step(s)
    assert out.num_computed[0] == 32 and out.block_tables[0][:2] == [b0, b1]
    assert out.block_tables[0][2] == b2                   # the unhashed head is reused
    # exhaust the pool: the hashed blocks are reallocated and the hit is gone
    hashes = S.request_block_hashes(prompt, B, 2)
    s.add_request(2, list(range(900, 900 + 12 * B - 1)), 1)
    _step(s)
    assert not set(hashes) & set(s.pool.cached)
    s.add_request(3, prompt, 1)
    out = _step(s)
    assert out.num_computed[0] == 0


def check_preemption_recompute():
    """[P1] §3.2 / [P4] §4.3: when the pool runs out, the newest running
    request is preempted: its blocks are freed, num_computed returns to 0 and
    it goes to the front of the waiting queue, later recomputing its tokens."""
    s = S.Scheduler(8, B, 256, 4, 512, enable_prefix_caching=False)
    s.add_request(0, list(range(64)), 100)                 # 4 full blocks
    s.add_request(1, list(range(100, 164)), 100)           # 4 full blocks
    _step(s)
    assert s.pool.num_free() == 0
    out = _step(s)                                        # both need a 5th block now
    assert out.preempted == [1] and out.request_ids == [0]
    r1 = s.requests[1]
    assert r1.num_computed == 0 and r1.blocks == [] and s.waiting[0] is r1
    assert s.total_preemptions == 1
    gen1 = r1.num_generated
    # request 0 finishes; request 1 comes back and recomputes prompt + output
    s.requests[0].max_new_tokens = s.requests[0].num_generated + 1
    _step(s)
    out = _step(s)
    assert out.request_ids == [1] and out.num_computed == [0]
    assert out.num_new == [64 + gen1]


def check_no_chunk_waits_for_budget():
    """[P4] §4.2 / [P1] §3.2: without chunked prefill a prompt that does not
    fit the remaining budget is not admitted in part."""
    s = S.Scheduler(100, B, 100, 8, 512, enable_chunked_prefill=False)
    s.add_request(0, list(range(60)), 5)
    s.add_request(1, list(range(200, 260)), 5)
    out = _step(s)
    assert out.request_ids == [0] and out.num_new == [60]
    out = _step(s)
    assert out.request_ids == [0, 1] and out.num_new == [1, 60]


def check_copy_on_write_fork():
    """[P1] §4.3.2: samples forked from one prompt share its blocks; the first
    sample to write into the shared partly filled block gets a copy, the
    last one writes in place; full prompt blocks stay shared."""
    s = S.Scheduler(30, B, 256, 8, 512)
    s.add_request(0, list(range(40)), 10)                 # blocks: 16 + 16 + 8
    _step(s)
    assert s.fork(0, 1, 10) and s.fork(0, 2, 10)
    shared = list(s.requests[0].blocks)
    assert all(s.pool.blocks[b].ref_cnt == 3 for b in shared)
    out = s.schedule()
    assert out.request_ids == [0, 1, 2]
    assert [src for src, _ in out.copies] == [shared[2], shared[2]]
    t = out.block_tables
    assert t[0][:2] == t[1][:2] == t[2][:2] == shared[:2]
    assert t[2][2] == shared[2] and len({t[0][2], t[1][2], t[2][2]}) == 3
    assert [dst for _, dst in out.copies] == [t[0][2], t[1][2]]
    s.update([1, 2, 3])
    s.check_invariants()
    # a prefilled request cannot fork before its prefill is done
    s.add_request(5, list(range(300)), 3)
    assert not s.fork(5, 6, 3)


def check_block_hash_chain():
    """[P4] §3.5: a block's hash depends on its tokens and on every earlier
    block (chained), not on where the block lives; only full blocks count."""
    rng = np.random.default_rng(0)
    toks = rng.integers(0, 32000, 5 * B)
    h = S.request_block_hashes(toks, B, 5)
    assert len(set(h)) == 5
    t2 = toks.copy()
    t2[2 * B + 3] += 1
    h2 = S.request_block_hashes(t2, B, 5)
    assert h2[:2] == h[:2] and all(a != b for a, b in zip(h2[2:], h[2:]))
    assert S.request_block_hashes(np.concatenate([toks, [1, 2, 3]]), B, 5) == h
    # same block content after a different prefix: different hash
    t3 = np.concatenate([toks[B:2 * B], toks[B:2 * B]])
    h3 = S.request_block_hashes(t3, B, 2)
    assert h3[0] != h3[1]


def check_random_trace_invariants():
    """Over a seeded trace with preemption pressure, forks and prefix hits:
    table membership equals ref counts; the free queue is exactly the
    unreferenced blocks; every step's tables cover its tokens and its slots
    are distinct; budget and sequence limits hold; every request finishes."""
    from workloads.trace import trace
    t = trace("sched_small")
    s = S.Scheduler(t.num_blocks, t.block_size, t.max_num_batched_tokens, t.max_num_seqs,
                    t.max_model_len)
    done, steps_with_copies, preempts = set(), 0, 0
    for step in range(t.num_steps):
        for rid, prompt, n in t.arrivals.get(step, []):
            s.add_request(rid, prompt, n)
        for parent, child, n in t.forks.get(step, []):
            s.fork(parent, child, n)
        out = s.schedule()
        assert out.num_tokens <= t.max_num_batched_tokens
        assert len(out.request_ids) <= t.max_num_seqs + sum(len(v) for v in t.forks.values())
        slots = []
        for c, n, tab in zip(out.num_computed, out.num_new, out.block_tables):
            assert len(tab) == -(-(c + n) // B)
            slots += [tab[p // B] * B + p % B for p in range(c, c + n)]
        assert len(set(slots)) == len(slots)
        steps_with_copies += bool(out.copies)
        preempts += len(out.preempted)
        sampled = [t.sampled(r, s.requests[r].num_generated) for r in out.request_ids]
        done |= set(s.update(sampled))
        s.check_invariants()
    assert done == set(s.requests), "trace did not drain"
    assert steps_with_copies > 0 and preempts > 0 and s.total_prefix_hit_tokens > 0


ALL_CHECKS = [
    check_chunk_sizes_worked_example,
    check_threshold_chunks,
    check_allocate_slots_block_count,
    check_new_block_on_len_mod_1,
    check_prefix_hit_sets_computed,
    check_shared_system_prompt_refcounts,
    check_free_queue_order_and_reuse,
    check_preemption_recompute,
    check_no_chunk_waits_for_budget,
    check_copy_on_write_fork,
    check_block_hash_chain,
    check_random_trace_invariants,
]
