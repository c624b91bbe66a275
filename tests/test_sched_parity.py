"""The library's C++ block manager / scheduler against the oracle, step by
step on seeded traces: every step's metadata, the finished requests, and the
whole internal state (free queue order, reference counts, hashes, per-request
progress) must be identical.  Host code only: runs without a GPU."""

import numpy as np
import pytest
import xxhash

from oracle import sched as S
from workloads.trace import TRACES, trace

pa = pytest.importorskip("paged_kv_attention_07_amd")
from paged_kv_attention_07_amd import sched as PS  # noqa: E402


def test_xxh64_matches_reference_library():
    """XXH64 written from the published specification agrees with the
    xxhash package (an independent implementation) on every length class:
    < 4, < 8, < 32 and multi-stripe inputs, with several seeds."""
    rng = np.random.default_rng(0)
    for n in list(range(0, 70)) + [71, 72, 100, 127, 128, 129, 1000, 4099]:
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        for seed in (0, 1, 0x9E3779B97F4A7C15, 2 ** 64 - 1):
            assert PS.xxh64(data, seed) == xxhash.xxh64_intdigest(data, seed), (n, seed)


def test_block_hash_matches_oracle():
    rng = np.random.default_rng(1)
    parent = None
    for _ in range(20):
        toks = rng.integers(0, 2 ** 31 - 1, 16)
        h = PS.block_hash(parent, toks)
        assert h == S.block_hash(parent, toks)
        parent = h


def _pair(t):
    kw = dict(num_blocks=t.num_blocks, block_size=t.block_size,
              max_num_batched_tokens=t.max_num_batched_tokens, max_num_seqs=t.max_num_seqs,
              max_model_len=t.max_model_len, enable_chunked_prefill=t.enable_chunked_prefill,
              enable_prefix_caching=t.enable_prefix_caching,
              long_prefill_token_threshold=t.long_prefill_token_threshold)
    return S.Scheduler(**kw), PS.Scheduler(**kw)


def _compare_state(o, c):
    assert c.free_queue() == o.pool.free
    for b in o.pool.blocks:
        assert c.block(b.block_id) == (b.ref_cnt, b.hash), b.block_id
    for rid, r in o.requests.items():
        info = c.request(rid)
        assert info["status"] == r.status, rid
        assert (info["num_tokens"], info["num_computed"], info["num_generated"],
                info["prompt_len"]) == (len(r.tokens), r.num_computed, r.num_generated,
                                        r.prompt_len), rid
        assert info["blocks"] == r.blocks, rid
    st = c.stats()
    assert st["num_free_blocks"] == len(o.pool.free)
    assert st["num_cached_blocks"] == len(o.pool.cached)
    assert st["num_running"] == len(o.running) and st["num_waiting"] == len(o.waiting)
    assert st["total_preemptions"] == o.total_preemptions
    assert st["total_prefix_hit_tokens"] == o.total_prefix_hit_tokens


@pytest.mark.parametrize("name", [n for n in TRACES if n.startswith("sched_")])
def test_scheduler_parity_on_trace(name):
    t = trace(name)
    o, c = _pair(t)
    events = {"copies": 0, "preempted": 0, "hits": 0, "forks": 0}
    for step in range(t.num_steps):
        for rid, prompt, n in t.arrivals.get(step, []):
            o.add_request(rid, prompt, n)
            c.add_request(rid, prompt, n)
        for parent, child, n in t.forks.get(step, []):
            a, b = o.fork(parent, child, n), c.fork(parent, child, n)
            assert a == b, (step, parent, child)
            events["forks"] += a
        ro, rc = o.schedule(), c.schedule()
        assert rc.request_ids.tolist() == ro.request_ids, step
        assert rc.num_new.tolist() == ro.num_new, step
        assert rc.num_computed.tolist() == ro.num_computed, step
        assert rc.seq_lens.tolist() == [a + b for a, b in zip(ro.num_computed, ro.num_new)]
        for i, tab in enumerate(ro.block_tables):
            row = rc.block_table[i]
            assert row[:len(tab)].tolist() == tab and np.all(row[len(tab):] == -1), (step, i)
        assert rc.token_ids.tolist() == ro.token_ids, step
        assert [tuple(p) for p in rc.copy_pairs.tolist()] == ro.copies, step
        assert rc.preempted.tolist() == ro.preempted, step
        if ro.request_ids:
            assert rc.max_query_len == max(ro.num_new)
        events["copies"] += len(ro.copies)
        events["preempted"] += len(ro.preempted)
        sampled = [t.sampled(r, o.requests[r].num_generated) for r in ro.request_ids]
        assert c.update(sampled) == o.update(sampled), step
        if step % 7 == 0 or ro.copies or ro.preempted:
            _compare_state(o, c)
    _compare_state(o, c)
    assert all(r.status == S.FINISHED for r in o.requests.values()), "trace did not drain"
    # the trace exercised what it was built for
    if name == "sched_small":
        assert events["copies"] and events["preempted"] and events["forks"]
        assert o.total_prefix_hit_tokens > 0
    if name == "sched_noprefix":
        assert events["preempted"] and o.total_prefix_hit_tokens == 0


def test_scheduler_errors():
    c = PS.Scheduler(8, 16, 64, 4, 128)
    c.add_request(1, [1, 2, 3], 4)
    with pytest.raises(pa.PAError):
        c.add_request(1, [1], 1)                     # duplicate id
    with pytest.raises(pa.PAError):
        c.add_request(2, [], 1)                      # empty prompt
    with pytest.raises(pa.PAError):
        c.add_request(3, list(range(100)), 40)       # past max_model_len
    with pytest.raises(pa.PAError):
        c.update([])                                 # update before schedule
    st = c.schedule()
    with pytest.raises(pa.PAError):
        c.schedule()                                 # schedule twice
    with pytest.raises(pa.PAError):
        c.update([1, 2])                             # wrong count
    assert c.update([5] * st.num_seqs) == []
    assert not c.fork(99, 100, 3)                    # unknown parent: no fork
    with pytest.raises(pa.PAError):
        PS.Scheduler(0, 16, 64, 4, 128)
