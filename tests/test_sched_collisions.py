"""Prefix caching when block hashes collide (CPU only).

With the block hash narrowed to 6 bits, unrelated blocks share a hash all the
time.  The property that matters is then checked directly: a step's requests
attend only to KV rows computed from their own tokens.  The test keeps a
model of what each block holds (every scheduled token written to its block
and offset, every copy-on-write pair applied) and, after each step's writes,
compares every position a scheduled request attends to with that request's
token at the position.  A scheduler that took a prefix-cache hit on the hash
alone would attach another prompt's rows; the planted variant below does
exactly that and must be caught.  The library's scheduler, built with the
same narrow hash, must still match the oracle step by step.
"""

import contextlib

import numpy as np
import pytest

import sched_build
from oracle import sched as S
from sched_build import CXX
from workloads.trace import TRACES, trace

MASK = 0x3F


@contextlib.contextmanager
def narrow_hash(mask=MASK):
    full = S.block_hash
    S.block_hash = lambda parent, tokens: full(parent, tokens) & mask
    try:
        yield
    finally:
        S.block_hash = full


def _hits_on_hash_alone(self, r):
    """Planted mistake: a cached hash is taken as a hit without comparing
    the block's token ids."""
    usable = (len(r.tokens) - 1) // self.B
    hits, parent = [], None
    for k in range(usable):
        parent = S.block_hash(parent, r.tokens[k * self.B:(k + 1) * self.B])
        bid = self.pool.cached.get(parent)
        if bid is None:
            break
        hits.append(bid)
    return hits


def run_with_content_model(t):
    """Drive the oracle scheduler through trace `t`, checking after every
    step that each scheduled request's visible KV rows hold its own tokens.
    Returns the prefix-hit token count."""
    kw = dict(num_blocks=t.num_blocks, block_size=t.block_size,
              max_num_batched_tokens=t.max_num_batched_tokens, max_num_seqs=t.max_num_seqs,
              max_model_len=t.max_model_len, enable_chunked_prefill=t.enable_chunked_prefill,
              enable_prefix_caching=t.enable_prefix_caching,
              long_prefill_token_threshold=t.long_prefill_token_threshold)
    o = S.Scheduler(**kw)
    B = t.block_size
    content = np.full((t.num_blocks, B), -1, np.int64)     # token whose K/V each row holds
    for step in range(t.num_steps):
        for rid, prompt, n in t.arrivals.get(step, []):
            o.add_request(rid, prompt, n)
        for parent, child, n in t.forks.get(step, []):
            o.fork(parent, child, n)
        out = o.schedule()
        for src, dst in out.copies:
            content[dst] = content[src]
        at = 0
        for i, rid in enumerate(out.request_ids):
            tab, nc, n = out.block_tables[i], out.num_computed[i], out.num_new[i]
            for j, tok in enumerate(out.token_ids[at:at + n]):
                p = nc + j
                content[tab[p // B], p % B] = tok
            at += n
        for i, rid in enumerate(out.request_ids):
            tab, L = out.block_tables[i], out.num_computed[i] + out.num_new[i]
            toks = np.asarray(o.requests[rid].tokens[:L], np.int64)
            pos = np.arange(L)
            held = content[np.asarray(tab)[pos // B], pos % B]
            bad = np.nonzero(held != toks)[0]
            assert bad.size == 0, (f"step {step}: request {rid} attends to rows of other tokens "
                                   f"at positions {bad[:8].tolist()}")
        o.update([t.sampled(r, o.requests[r].num_generated) for r in out.request_ids])
    assert all(r.status == S.FINISHED for r in o.requests.values()), "trace did not drain"
    return o.total_prefix_hit_tokens


@pytest.mark.parametrize("name", ["sched_small", "sched_nochunk"])
def test_full_hash_keeps_rows_consistent(name):
    assert run_with_content_model(trace(name)) > 0


@pytest.mark.parametrize("name", ["sched_small", "sched_nochunk"])
def test_narrow_hash_keeps_rows_consistent(name):
    with narrow_hash():
        hits = run_with_content_model(trace(name))
    assert hits > 0            # true shared prefixes still hit


def test_hits_on_hash_alone_are_caught(monkeypatch):
    monkeypatch.setattr(S.Scheduler, "_prefix_hits", _hits_on_hash_alone)
    with narrow_hash(), pytest.raises(AssertionError, match="attends to rows of other tokens"):
        run_with_content_model(trace("sched_small"))


@pytest.mark.skipif(CXX is None, reason="needs the host C++ compiler")
def test_library_scheduler_matches_oracle_under_narrow_hash(tmp_path):
    lib = sched_build.build(tmp_path / "libpa_sched_narrow.so",
                            [f"-DPA_SCHED_HASH_MASK={MASK:#x}"])
    prelude = f"""
        from oracle import sched as S
        _full = S.block_hash
        S.block_hash = lambda parent, tokens: _full(parent, tokens) & {MASK:#x}
    """
    r = sched_build.run_parity_child(lib, tmp_path, prelude=prelude)
    assert r.returncode == 0 and "passed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
