"""Plain-Python oracle of the host-side KV block manager and step scheduler.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and by nothing in the product).
The C++ scheduler in the library is checked against it step by step.

Sources (web pages, cited by title and section):
  [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成"
  [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
  [P3] the nano-vllm code walk-through on blog.mospan.cn (its title is not
       in the extracted text), section "块管理器"
  [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"

What it models.
  * Blocks carry a reference count and, once full and computed, a content
    hash ([P4] §3.3 KVCacheBlock).  Blocks with ref_cnt 0 sit in one free
    queue: blocks without a hash at the head, hashed ones (prefix-cache
    candidates) at the tail; allocation takes from the head ([P4] §3.3,
    §3.6 step 4).  Taking a hashed block for new content evicts its hash.
  * Block hash of logical block k = H(hash of block k-1, token ids of block
    k), over full blocks only ([P4] §3.5; [P2] §3.6 step 2).  H is XXH64
    ([P3] names xxhash64) over the parent hash as 8 little-endian bytes
    (omitted for block 0) followed by the block's token ids as 4-byte
    little-endian integers.
  * Prefix lookup walks a request's full blocks in order and stops at the
    first miss ([P4] §3.5 get_computed_blocks); a hit sets num_computed to
    hits * block_size ([P4] §3.5) and takes a reference on each hit block,
    pulling it out of the free queue if it was free ([P2] §3.6).
  * One step ([P4] §4.2; [P2] §3.3; [P1] §3.2): the token budget is shared;
    running requests first (each min(remaining, threshold, budget,
    max_model_len - computed) new tokens, allocate_slots, preempt the newest
    running request on failure ([P1] §3.2 FCFS preemption; [P4] §4.3: free
    its blocks, num_computed = 0, back to the front of waiting)); then
    waiting requests in order while budget and sequence slots remain.
  * allocate_slots: ceil((computed + new) / block_size) blocks in total, the
    missing ones from the free queue head ([P2] §3.3); none if the pool
    cannot cover them.
  * Copy-on-write ([P1] §4.3.2): a block this step writes into that is
    shared (ref_cnt > 1) is first copied to a fresh block, which replaces it
    in the writer's table; the copy is reported as a (src, dst) pair.
  * After the step ([P4] §3.6 step 4): computed counts advance; a request
    whose computed count reaches its token count samples one token (given
    as input); full computed blocks are hashed and registered; finished
    requests free their blocks, last block first: hashed ones to the queue
    tail, others to the head.

Readings of points the pages leave open (each also listed in the design
notes): at least one prompt token is always computed, so a full-prompt hit
keeps its last block out of the hit list; without chunked prefill a waiting
request that does not fit stops admission for the step ([P4] §4.2's break;
[P1] §3.2 shows a skip instead); waiting requests are not admitted in a step
that preempted; a prefix-cache hit needs the hash and the cached block's own
token ids to match (two blocks whose hashes collide are never taken for one
another; the chain itself is followed through the hashes); a hash that is
already registered keeps its first block.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np
import xxhash

WAITING, RUNNING, FINISHED = "waiting", "running", "finished"


def block_hash(parent: Optional[int], tokens) -> int:
    """[P4] §3.5 chained block hash with XXH64 ([P3]), seed 0."""
    h = xxhash.xxh64(seed=0)
    if parent is not None:
        h.update(int(parent).to_bytes(8, "little"))
    h.update(np.asarray(tokens, dtype="<i4").tobytes())
    return h.intdigest()


def request_block_hashes(tokens, block_size: int, count: int) -> List[int]:
    """Hashes of the first `count` full blocks of a token sequence."""
    out: List[int] = []
    parent = None
    for k in range(count):
        parent = block_hash(parent, tokens[k * block_size:(k + 1) * block_size])
        out.append(parent)
    return out


@dataclasses.dataclass
class Block:
    block_id: int
    ref_cnt: int = 0
    hash: Optional[int] = None
    tokens: Optional[Tuple[int, ...]] = None   # token ids, kept while the block is hashed


@dataclasses.dataclass
class Request:
    request_id: int
    tokens: List[int]
    prompt_len: int
    max_new_tokens: int
    num_generated: int = 0
    num_computed: int = 0
    blocks: List[int] = dataclasses.field(default_factory=list)
    status: str = WAITING
    prefix_hit_tokens: int = 0


@dataclasses.dataclass
class StepOutput:
    request_ids: List[int]
    num_new: List[int]
    num_computed: List[int]          # before the step
    block_tables: List[List[int]]    # after allocation (and copy-on-write)
    token_ids: List[int]             # the step's input tokens, request by request
    copies: List[Tuple[int, int]]    # (src, dst) block copies to run first
    preempted: List[int]

    @property
    def num_tokens(self) -> int:
        return int(sum(self.num_new))


class BlockPool:
    """Blocks, the free queue (a Python list: index 0 is the head) and the
    prefix-cache map from hash to block id."""

    def __init__(self, num_blocks: int):
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.free: List[int] = list(range(num_blocks))
        self.cached: Dict[int, int] = {}

    def num_free(self) -> int:
        return len(self.free)

    def take_fresh(self) -> int:
        """Pop the head of the free queue for new content (evicting its hash)."""
        b = self.blocks[self.free.pop(0)]
        if b.hash is not None:
            if self.cached.get(b.hash) == b.block_id:
                del self.cached[b.hash]
            b.hash = None
            b.tokens = None
        b.ref_cnt = 1
        return b.block_id

    def take_cached(self, block_id: int) -> None:
        """Reference a prefix-cache hit, pulling it out of the free queue."""
        b = self.blocks[block_id]
        if b.ref_cnt == 0:
            self.free.remove(block_id)
        b.ref_cnt += 1

    def release(self, block_ids: List[int]) -> None:
        for bid in reversed(block_ids):
            b = self.blocks[bid]
            b.ref_cnt -= 1
            assert b.ref_cnt >= 0
            if b.ref_cnt == 0:
                if b.hash is None:
                    self.free.insert(0, bid)
                else:
                    self.free.append(bid)


class Scheduler:
    def __init__(self, num_blocks: int, block_size: int, max_num_batched_tokens: int,
                 max_num_seqs: int, max_model_len: int, enable_chunked_prefill: bool = True,
                 enable_prefix_caching: bool = True, long_prefill_token_threshold: int = 0):
        self.B = block_size
        self.budget = max_num_batched_tokens
        self.max_num_seqs = max_num_seqs
        self.max_model_len = max_model_len
        self.chunked = enable_chunked_prefill
        self.prefix = enable_prefix_caching
        self.threshold = long_prefill_token_threshold
        self.pool = BlockPool(num_blocks)
        self.requests: Dict[int, Request] = {}
        self.running: List[Request] = []
        self.waiting: List[Request] = []
        self.last: Optional[StepOutput] = None
        self.total_preemptions = 0
        self.total_prefix_hit_tokens = 0

    # ---- requests -------------------------------------------------------
    def add_request(self, request_id: int, prompt, max_new_tokens: int) -> None:
        assert request_id not in self.requests and len(prompt) > 0 and max_new_tokens > 0
        # the last sampled token is never written: positions stay < max_model_len
        assert len(prompt) + max_new_tokens - 1 <= self.max_model_len
        r = Request(request_id, [int(t) for t in prompt], len(prompt), max_new_tokens)
        self.requests[request_id] = r
        self.waiting.append(r)

    def fork(self, parent_id: int, child_id: int, max_new_tokens: int) -> bool:
        """[P1] §4.3.2: a new sample of a running request shares all of its
        blocks (one more reference each) and continues from the same tokens.
        Only a request past its prefill (every token but the last sampled one
        computed) can fork, and only while fewer than max_num_seqs requests
        run; otherwise nothing happens and False is returned."""
        p = self.requests.get(parent_id)
        assert child_id not in self.requests
        if (p is None or p.status != RUNNING or p.num_computed != len(p.tokens) - 1
                or p.num_generated >= max_new_tokens
                or len(self.running) >= self.max_num_seqs):
            return False
        assert p.prompt_len + max_new_tokens - 1 <= self.max_model_len
        c = Request(child_id, list(p.tokens), p.prompt_len, max_new_tokens,
                    num_generated=p.num_generated, num_computed=p.num_computed,
                    blocks=list(p.blocks), status=RUNNING)
        for bid in c.blocks:
            self.pool.blocks[bid].ref_cnt += 1
        self.requests[child_id] = c
        self.running.append(c)
        return True

    # ---- one step -------------------------------------------------------
    def _cap(self, computed: int, num_new: int, budget: int) -> int:
        """[P1] §3.2: chunk threshold, remaining budget, model length."""
        if 0 < self.threshold < num_new:
            num_new = self.threshold
        num_new = min(num_new, budget)
        return min(num_new, self.max_model_len - computed)

    def _allocate_slots(self, r: Request, num_new: int, copies) -> bool:
        need_total = -(-(r.num_computed + num_new) // self.B)
        need_new = need_total - len(r.blocks)
        shared = [j for j in range(r.num_computed // self.B, len(r.blocks))
                  if self.pool.blocks[r.blocks[j]].ref_cnt > 1]
        if self.pool.num_free() < need_new + len(shared):
            return False
        for j in shared:                      # copy-on-write
            src = r.blocks[j]
            dst = self.pool.take_fresh()
            self.pool.blocks[src].ref_cnt -= 1
            r.blocks[j] = dst
            copies.append((src, dst))
        for _ in range(need_new):
            r.blocks.append(self.pool.take_fresh())
        return True

    def _preempt(self, r: Request) -> None:
        self.pool.release(r.blocks)
        r.blocks = []
        r.num_computed = 0
        r.status = WAITING
        self.waiting.insert(0, r)
        self.total_preemptions += 1

    def _prefix_hits(self, r: Request) -> List[int]:
        usable = (len(r.tokens) - 1) // self.B          # keep >= 1 token to compute
        hits: List[int] = []
        parent = None
        for k in range(usable):
            parent = block_hash(parent, r.tokens[k * self.B:(k + 1) * self.B])
            bid = self.pool.cached.get(parent)
            if bid is None or self.pool.blocks[bid].tokens != tuple(
                    r.tokens[k * self.B:(k + 1) * self.B]):
                break
            hits.append(bid)
        return hits

    def schedule(self) -> StepOutput:
        budget = self.budget
        sched: List[Tuple[Request, int, int]] = []   # (request, computed before, new)
        copies: List[Tuple[int, int]] = []
        preempted: List[int] = []
        i = 0
        while i < len(self.running) and budget > 0:
            r = self.running[i]
            num_new = self._cap(r.num_computed, len(r.tokens) - r.num_computed, budget)
            if num_new <= 0:
                i += 1
                continue
            while not self._allocate_slots(r, num_new, copies):
                victim = self.running.pop()
                self._preempt(victim)
                preempted.append(victim.request_id)
                if victim is r:
                    r = None
                    break
            if r is None:
                break
            sched.append((r, r.num_computed, num_new))
            budget -= num_new
            i += 1
        if not preempted:
            while self.waiting and budget > 0 and len(self.running) < self.max_num_seqs:
                r = self.waiting[0]
                hits = self._prefix_hits(r) if (self.prefix and r.num_computed == 0) else []
                start = len(hits) * self.B
                remaining = len(r.tokens) - start
                num_new = self._cap(start, remaining, budget)
                if num_new <= 0 or (not self.chunked and num_new < remaining):
                    break
                need_new = -(-(start + num_new) // self.B) - len(hits)
                free_hits = sum(1 for b in hits if self.pool.blocks[b].ref_cnt == 0)
                if self.pool.num_free() - free_hits < need_new:
                    break
                for b in hits:
                    self.pool.take_cached(b)
                r.blocks = list(hits)
                r.num_computed = start
                r.prefix_hit_tokens += start
                self.total_prefix_hit_tokens += start
                for _ in range(need_new):
                    r.blocks.append(self.pool.take_fresh())
                self.waiting.pop(0)
                r.status = RUNNING
                self.running.append(r)
                sched.append((r, start, num_new))
                budget -= num_new
        out = StepOutput(
            request_ids=[r.request_id for r, _, _ in sched],
            num_new=[n for _, _, n in sched],
            num_computed=[c for _, c, _ in sched],
            block_tables=[list(r.blocks) for r, _, _ in sched],
            token_ids=[t for r, c, n in sched for t in r.tokens[c:c + n]],
            copies=copies, preempted=preempted)
        self._sched = sched
        self.last = out
        return out

    def update(self, sampled: List[int]) -> List[int]:
        """Advance the scheduled requests; sampled[i] is the token request i
        of the last step samples if the step reached its sequence end.
        Returns the ids of requests that finished."""
        finished: List[int] = []
        for (r, before, n), tok in zip(self._sched, sampled):
            if r.status != RUNNING:
                continue
            r.num_computed = before + n
            if r.num_computed == len(r.tokens):
                r.tokens.append(int(tok))
                r.num_generated += 1
                if r.num_generated >= r.max_new_tokens:
                    r.status = FINISHED
            if self.prefix:
                self._cache_blocks(r)
        for r, _, _ in self._sched:
            if r.status == FINISHED and r.blocks:
                self.running.remove(r)
                self.pool.release(r.blocks)
                r.blocks = []
                finished.append(r.request_id)
        self._sched = []
        return finished

    def _cache_blocks(self, r: Request) -> None:
        full = r.num_computed // self.B
        hashes = request_block_hashes(r.tokens, self.B, full)
        for k in range(full):
            b = self.pool.blocks[r.blocks[k]]
            if b.hash is None:
                b.hash = hashes[k]
                b.tokens = tuple(r.tokens[k * self.B:(k + 1) * self.B])
                self.pool.cached.setdefault(hashes[k], b.block_id)

    # ---- invariants ------------------------------------------------------
    def check_invariants(self) -> None:
        refs = np.zeros(len(self.pool.blocks), np.int64)
        for r in self.requests.values():
            for b in r.blocks:
                refs[b] += 1
        got = np.array([b.ref_cnt for b in self.pool.blocks])
        assert np.array_equal(refs, got), "ref counts differ from table membership"
        free = set(self.pool.free)
        assert len(free) == len(self.pool.free)
        assert free == {b.block_id for b in self.pool.blocks if b.ref_cnt == 0}
        for h, bid in self.pool.cached.items():
            assert self.pool.blocks[bid].hash == h
