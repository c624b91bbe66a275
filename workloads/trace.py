"""Seeded synthetic serving traces for the block manager / scheduler.

Only inputs live here (prompts, arrival steps, output lengths, forks and the
tokens each request "samples"); none of the scheduler's arithmetic.  Sampled
tokens come from a counter-based generator (SplitMix64 of the request id and
the index of the generated token), so any implementation can draw the same
token for the same request and step without shared state.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 finaliser (Steele, Lea and Flood, 2014)."""
    x = (x + 0x9E3779B97F4A7C15) & _M64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _M64
    return x ^ (x >> 31)


def sampled_token(seed: int, request_id: int, index: int, vocab: int) -> int:
    """Token that request `request_id` samples as its `index`-th output."""
    return splitmix64(((seed & 0xFFFF) << 48) ^ (request_id << 20) ^ index) % vocab


@dataclasses.dataclass
class Trace:
    name: str
    seed: int
    vocab: int
    block_size: int
    num_blocks: int
    max_num_batched_tokens: int
    max_num_seqs: int
    max_model_len: int
    # step -> [(request_id, prompt, max_new_tokens)]
    arrivals: Dict[int, List[Tuple[int, np.ndarray, int]]]
    # step -> [(parent_id, child_id, max_new_tokens)]
    forks: Dict[int, List[Tuple[int, int, int]]]
    num_steps: int
    enable_chunked_prefill: bool = True
    enable_prefix_caching: bool = True
    long_prefill_token_threshold: int = 0

    def sampled(self, request_id: int, index: int) -> int:
        return sampled_token(self.seed, request_id, index, self.vocab)


def make_trace(name: str, *, seed: int, num_requests: int, num_steps: int, num_blocks: int,
               max_num_batched_tokens: int, max_num_seqs: int, max_model_len: int,
               prompt_len: Tuple[int, int], max_new: Tuple[int, int], num_prefixes: int = 4,
               prefix_len: Tuple[int, int] = (16, 200), prefix_share: float = 0.6,
               arrival_steps: int = 0, fork_prob: float = 0.0, fork_n: int = 3,
               vocab: int = 32000, block_size: int = 16, **flags) -> Trace:
    """Requests with uniform prompt / output lengths; a share of them start
    with one of a few shared system prompts (prefix-cache hits); arrivals
    spread uniformly over the first `arrival_steps` steps (0 = all at step 0);
    some requests fork into `fork_n` samples a few steps after arriving."""
    rng = np.random.default_rng(seed)
    prefixes = [rng.integers(0, vocab, rng.integers(prefix_len[0], prefix_len[1] + 1))
                for _ in range(num_prefixes)]
    arrivals: Dict[int, list] = {}
    forks: Dict[int, list] = {}
    next_id = 0
    for _ in range(num_requests):
        rid = next_id
        next_id += 1
        L = int(rng.integers(prompt_len[0], prompt_len[1] + 1))
        if num_prefixes and rng.random() < prefix_share:
            pre = prefixes[int(rng.integers(num_prefixes))][:L - 1]
            prompt = np.concatenate([pre, rng.integers(0, vocab, L - pre.size)])
        else:
            prompt = rng.integers(0, vocab, L)
        n_out = int(rng.integers(max_new[0], max_new[1] + 1))
        n_out = max(1, min(n_out, max_model_len + 1 - L))
        step = int(rng.integers(0, arrival_steps)) if arrival_steps else 0
        arrivals.setdefault(step, []).append((rid, prompt.astype(np.int32), n_out))
        if fork_prob and rng.random() < fork_prob and n_out > 4:
            fstep = step + int(rng.integers(2, 6))
            for _ in range(fork_n - 1):
                forks.setdefault(fstep, []).append((rid, next_id, n_out))
                next_id += 1
    return Trace(name=name, seed=seed, vocab=vocab, block_size=block_size, num_blocks=num_blocks,
                 max_num_batched_tokens=max_num_batched_tokens, max_num_seqs=max_num_seqs,
                 max_model_len=max_model_len, arrivals=arrivals, forks=forks,
                 num_steps=num_steps, **flags)


TRACES = {
    # small: oracle-speed parity over many steps, with preemption pressure
    "sched_small": dict(seed=3001, num_requests=40, num_steps=400, num_blocks=40,
                        max_num_batched_tokens=64, max_num_seqs=12, max_model_len=512,
                        prompt_len=(5, 120), max_new=(1, 60), arrival_steps=60,
                        fork_prob=0.2),
    "sched_nochunk": dict(seed=3002, num_requests=30, num_steps=300, num_blocks=48,
                          max_num_batched_tokens=128, max_num_seqs=8, max_model_len=512,
                          prompt_len=(5, 100), max_new=(1, 40), arrival_steps=40,
                          enable_chunked_prefill=False),
    "sched_noprefix": dict(seed=3003, num_requests=30, num_steps=300, num_blocks=36,
                           max_num_batched_tokens=48, max_num_seqs=10, max_model_len=512,
                           prompt_len=(5, 90), max_new=(1, 50), arrival_steps=50,
                           enable_prefix_caching=False, long_prefill_token_threshold=20),
    # serving-shaped: Llama-3-8B layer, 2048-token budget, system prompts
    "serve_llama3_2k": dict(seed=3101, num_requests=256, num_steps=600, num_blocks=20000,
                            max_num_batched_tokens=2048, max_num_seqs=128, max_model_len=4096,
                            prompt_len=(64, 1536), max_new=(16, 256), num_prefixes=8,
                            prefix_len=(256, 1024), prefix_share=0.5, arrival_steps=60,
                            fork_prob=0.05),
}


TRACES["engine_small"] = dict(TRACES["sched_small"], seed=3201, num_requests=36)


def trace(name: str) -> Trace:
    return make_trace(name, **TRACES[name])


def step_inputs(seed: int, step: int, num_tokens: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, dtype: str):
    """q [T, Hq, D], k / v [T, Hkv, D] storage bits for one engine step (the
    stand-ins for a model's projections), seeded by (seed, step)."""
    from .gen import _normal
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x57E9, step]))
    return (_normal(rng, (num_tokens, num_q_heads, head_dim), dtype),
            _normal(rng, (num_tokens, num_kv_heads, head_dim), dtype),
            _normal(rng, (num_tokens, num_kv_heads, head_dim), dtype))
