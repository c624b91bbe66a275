"""Benchmark of the paged-KV-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--extra] [--only decode|mixed|prefix|long] [--splits S]
                    [--separate]

A step is one pass of the whole path over one batch: slot mapping of the new
tokens, reshape_and_cache of their K/V, then attention (decode for the decode
batch, mixed for the chunked-prefill batch).  By default the three run as one
attention launch (pa_cache_and_attend_*: the launch stores the new tokens and
reads them from the input rows) plus the split merge; --separate times the
three calls one after the other.  The shared-prefix leg always runs them
apart (its entry takes the cache as written).  Inputs are resident in HBM
before timing starts; several copies of the KV pool are rotated so that
successive steps do not hit in the 256 MB Infinity Cache.

Headline (`value`): algorithmic HBM bytes per decode step / step time, on the
64-request Llama-3-8B-layer decode batch.  Also reported: tokens/s of the
mixed chunked-prefill step, the roofline of the attention call (HIP events on
the launch stream), and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode HBM GB/s (% peak) + mixed-step tokens/sec, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "decode": "decode_bf16_64req",
    "mixed": "mixed_chunked_prefill_bf16",
    "prefix": "prefix_shared_decode_bf16",
    "long": "long_context_decode_bf16",
    "chunk": "prefill_chunk_bf16",
    "prefixplain": "prefix_shared_decode_bf16",
    "prefill2k": "prefill_chunk_2048_bf16",
    "prefill8k": "prefill_8192_bf16",
    "prefillbatch": "prefill_batch_4x1024_bf16",
}

DESCR = {
    "decode_bf16_64req": "Llama-3-8B layer decode (Hq 32, Hkv 8, D 128, bf16, block 16): 64 requests, "
                         "seq_len ~ U[512,4096], pool 20000 blocks, 1 new token each",
    "mixed_chunked_prefill_bf16": "Llama-3-8B layer chunked-prefill step: 512-token chunk on 1024 cached, "
                                  "2 x 10-token prefills, 61 decodes at 2048 (593 query tokens)",
    "prefix_shared_decode_bf16": "Llama-3-8B layer decode, 256 requests sharing a 1024-token prefix "
                                 "(64 blocks) + private suffix U[64,512]",
    "long_context_decode_bf16": "Llama-3-8B layer decode, 16 requests at 32768 tokens, pool 36000 blocks",
    "prefill_chunk_bf16": "Llama-3-8B layer prefill chunk alone: 512 new tokens on 1024 cached",
    "prefill_chunk_2048_bf16": "Llama-3-8B layer prefill: 2048 new tokens on 2048 cached",
    "prefill_8192_bf16": "Llama-3-8B layer prefill: fresh 8192-token prompt",
    "prefill_batch_4x1024_bf16": "Llama-3-8B layer prefill: 4 requests x ~1024-token chunks",
}


# --------------------------------------------------------------------------
# algorithmic byte / flop counts (what the method itself must move)
# --------------------------------------------------------------------------


def alg_counts(w):
    """Bytes each part of one step must move, and the attention's flops."""
    esz = 4 if w.dtype == "f32" else 2
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    T, R = w.num_tokens, w.num_seqs
    kb = 2 * Hkv * D * esz                       # K+V bytes per token per layer
    ql = w.q_lens
    rows = ql > 0
    keys_read = int(w.seq_lens[rows].astype(np.int64).sum())
    # unique KV bytes: shared physical blocks counted once
    used_tokens = 0
    seen = set()
    for r in np.nonzero(rows)[0]:
        L = int(w.seq_lens[r])
        nb = -(-L // B)
        for j in range(nb):
            blk = int(w.block_table[r, j])
            n_tok = min(B, L - j * B)
            if blk in seen:
                continue
            seen.add(blk)
            used_tokens += n_tok
    nblocks = int(sum(-(-int(L) // B) for L in w.seq_lens[rows]))
    attn_bytes_logical = keys_read * kb + 2 * T * Hq * D * esz + nblocks * 4 + R * 4 * 3
    attn_bytes_unique = used_tokens * kb + 2 * T * Hq * D * esz + nblocks * 4 + R * 4 * 3
    scatter_bytes = 2 * T * kb + T * 8
    slot_bytes = T * 4 + R * 8 + T * 8
    # flops: 4*D per (query head, visible key) pair (QK^T and PV)
    pairs = 0
    for r in np.nonzero(rows)[0]:
        c, n = int(w.num_computed[r]), int(ql[r])
        pairs += n * c + n * (n + 1) // 2
    flops = 4 * D * Hq * pairs
    chunk_pairs = 0
    for r in np.nonzero(ql > 1)[0]:
        c, n = int(w.num_computed[r]), int(ql[r])
        chunk_pairs += n * c + n * (n + 1) // 2
    return dict(attn_logical=attn_bytes_logical, attn_unique=attn_bytes_unique,
                scatter=scatter_bytes, slots=slot_bytes, flops=flops,
                chunk_flops=4 * D * Hq * chunk_pairs, kv_bytes_per_token=kb)


# --------------------------------------------------------------------------
# GPU side
# --------------------------------------------------------------------------


class Stepper:
    """Device copies of one workload and the step of the hot path over them."""

    def __init__(self, w, rotations: int, splits: int, shared_prefix: int = 0,
                 fused: bool = True):
        import torch
        import paged_kv_attention_07_amd as pa
        self.pa, self.torch, self.w, self.splits = pa, torch, w, splits
        self.fused = fused and not shared_prefix
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]

        def dev(a):
            if w.dtype == "f32":
                return torch.from_numpy(np.ascontiguousarray(a)).cuda()
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

        base = dev(w.pool)
        self.pools = [base] + [base.clone() for _ in range(rotations - 1)]
        self.q, self.kn, self.vn = dev(w.q), dev(w.k_new), dev(w.v_new)
        self.bt, self.sl = i32(w.block_table), i32(w.seq_lens)
        self.qsl, self.nc = i32(w.query_start_loc), i32(w.num_computed)
        self.out = torch.empty_like(self.q)
        self.slots = torch.empty(w.num_tokens, dtype=torch.int64, device="cuda")
        nbytes = pa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads,
                                                w.num_kv_heads, w.head_dim, w.max_seq_len,
                                                w.max_query_len, splits)
        self.shared_prefix = shared_prefix
        if shared_prefix:
            nbytes = max(nbytes, pa.pa_attention_decode_shared_prefix_workspace_size(
                w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_seq_len,
                shared_prefix, splits))
        self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        self.decode = w.is_decode_only

    def attention(self, kv):
        w, pa = self.w, self.pa
        if self.decode and self.shared_prefix:
            pa.pa_attention_decode_shared_prefix(
                self.q, kv, self.bt, self.sl, w.scale, w.max_seq_len, self.shared_prefix,
                out=self.out, workspace=self.ws, num_splits=self.splits)
        elif self.decode:
            pa.pa_attention_decode(self.q, kv, self.bt, self.sl, w.scale, w.max_seq_len,
                                   out=self.out, workspace=self.ws, num_splits=self.splits)
        else:
            pa.pa_attention_mixed(self.q, kv, self.bt, self.sl, self.qsl, self.nc, w.scale,
                                  w.max_query_len, w.max_seq_len, out=self.out,
                                  workspace=self.ws, num_splits=self.splits)

    def capture(self):
        """Capture the one-launch step over each pool copy in its own HIP
        graph (kernels only: the entry points allocate and synchronise
        nothing); `step` then replays them."""
        torch = self.torch
        assert self.fused, "graph replay covers the one-launch step"
        self.graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(self.pools)):
                self._fused(self.pools[i])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for kv in self.pools:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._fused(kv)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def _fused(self, kv):
        pa, w = self.pa, self.w
        if self.decode:
            pa.pa_cache_and_attend_decode(self.q, self.kn, self.vn, kv, self.bt, self.sl,
                                          w.scale, w.max_seq_len, out=self.out,
                                          slot_mapping=self.slots, workspace=self.ws,
                                          num_splits=self.splits)
        else:
            pa.pa_cache_and_attend_mixed(self.q, self.kn, self.vn, kv, self.bt, self.sl,
                                         self.qsl, self.nc, w.scale, w.max_query_len,
                                         w.max_seq_len, out=self.out,
                                         slot_mapping=self.slots, workspace=self.ws,
                                         num_splits=self.splits)

    def step(self, i, ev=None):
        pa, w = self.pa, self.w
        kv = self.pools[i % len(self.pools)]
        if getattr(self, "graphs", None):
            if ev is not None:
                ev[0].record()
            self.graphs[i % len(self.graphs)].replay()
            if ev is not None:
                ev[1].record()
            return
        if self.fused:
            if ev is not None:
                ev[0].record()
            if self.decode:
                pa.pa_cache_and_attend_decode(self.q, self.kn, self.vn, kv, self.bt, self.sl,
                                              w.scale, w.max_seq_len, out=self.out,
                                              slot_mapping=self.slots, workspace=self.ws,
                                              num_splits=self.splits)
            else:
                pa.pa_cache_and_attend_mixed(self.q, self.kn, self.vn, kv, self.bt, self.sl,
                                             self.qsl, self.nc, w.scale, w.max_query_len,
                                             w.max_seq_len, out=self.out,
                                             slot_mapping=self.slots, workspace=self.ws,
                                             num_splits=self.splits)
            if ev is not None:
                ev[1].record()
            return
        pa.pa_compute_slot_mapping(self.bt, self.qsl, self.nc, w.num_tokens, w.block_size,
                                   out=self.slots)
        pa.pa_reshape_and_cache(self.kn, self.vn, kv, self.slots)
        if ev is not None:
            ev[0].record()
        self.attention(kv)
        if ev is not None:
            ev[1].record()

    def run_flushed(self, launches: int, flush_bytes: int = 512 << 20):
        """Cold-cache launches: before each step a `flush_bytes` write and then
        a read of another `flush_bytes` buffer evict L2 and the 256 MB
        Infinity Cache (the read pass also takes the write-backs of the
        write, which would otherwise land inside the timed launch); HIP
        events bracket the attention call alone.  Returns the per-launch
        durations (ms)."""
        torch = self.torch
        scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
        other = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
        ms = []
        for i in range(launches):
            scratch.fill_(i & 0xFF)
            other.sum()
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            self.step(i, ev)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        del scratch, other
        return ms

    def run(self, steps: int, warmup: int, event_every: int = 1):
        """Time `steps` steps; the attention call of every `event_every`-th
        step is bracketed by HIP events on the launch stream (an event record
        between two launches leaves the GPU idle for a moment, so sampling
        keeps that measurement cost out of most steps)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        sampled = [i for i in range(steps) if i % max(1, event_every) == 0]
        events = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for i in sampled}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i, events.get(i))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        attn_ms = [a.elapsed_time(b) for a, b in events.values()]
        return (t1 - t0) * 1e3 / steps, attn_ms


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    passes (profiles/traffic.json), or None if the kernel's sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["hbm_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def gpu_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", ""),
            "cus": p.multi_processor_count, "hbm_gb": round(p.total_memory / 2**30, 1)}


def copy_reference(nbytes: int = 1 << 30, reps: int = 10):
    """Achievable-HBM reference: a device-to-device copy of `nbytes` (read +
    write counted), median of `reps` event-timed copies."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    t = float(np.median(ms)) * 1e-3
    return {"kind": "device-to-device copy (torch), read + write bytes / median time",
            "bytes": 2 * nbytes, "gbs": round(2 * nbytes / t / 1e9, 1),
            "pct_peak_hbm": round(100 * 2 * nbytes / t / 1e9 / HBM_PEAK_GBS, 2)}


# --------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# --------------------------------------------------------------------------


def cpu_baseline(w, budget_s: float = 12.0):
    """Time the oracle (as it stands, BLAS limited to one thread) on the
    first n requests of the same batch, n chosen so the run takes about
    `budget_s`; scaled to the same unit as the GPU figure (GB/s of
    algorithmic attention bytes)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        if ctx is not None:
            ctx.__enter__()
        slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size)
        t0 = time.perf_counter()
        pool = oracle.reshape_and_cache(w.pool, w.k_new, w.v_new, slots)
        t_scatter = time.perf_counter() - t0
        order = [r for r in range(w.num_seqs) if w.q_lens[r] > 0]
        # requests one at a time, in batch order, until the time budget is used
        sample, t_attn = [], 0.0
        for r in order:
            t0 = time.perf_counter()
            oracle.paged_attention(w.q, pool, w.block_table, w.seq_lens, w.query_start_loc,
                                   w.num_computed, w.scale, w.dtype, requests=[r])
            t_attn += time.perf_counter() - t0
            sample.append(r)
            if t_attn >= budget_s:
                break
        n = len(sample)
        passes = 1
        if n == len(order):
            # the whole batch fit the budget: time more full passes, keep the best
            best, spent = t_attn, t_attn
            while passes < 3 and spent + best < budget_s:
                t0 = time.perf_counter()
                oracle.paged_attention(w.q, pool, w.block_table, w.seq_lens,
                                       w.query_start_loc, w.num_computed, w.scale, w.dtype,
                                       requests=order)
                dt = time.perf_counter() - t0
                best, spent, passes = min(best, dt), spent + dt, passes + 1
            t_attn = best
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    esz = 4 if w.dtype == "f32" else 2
    kb = 2 * w.num_kv_heads * w.head_dim * esz
    keys = int(sum(int(w.seq_lens[r]) for r in sample))
    toks = int(sum(int(w.q_lens[r]) for r in sample))
    byts = keys * kb + 2 * toks * w.num_q_heads * w.head_dim * esz
    # scatter of the sample's tokens is charged pro rata
    t_total = t_attn + t_scatter * toks / max(1, w.num_tokens)
    return {
        "value": round(byts / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{n} of {len(order)} requests of {w.name} (slot mapping excluded, "
                  f"scatter charged pro rata): {toks} query tokens, {keys} keys, "
                  f"{t_total:.2f} s fp64 numpy, BLAS 1 thread"
                  + (f", best of {passes} full passes" if passes > 1 else ""),
        "tokens_per_s": round(toks / t_total, 3),
        "cpu": platform.processor() or platform.machine(),
        "host_cores_available": len(os.sched_getaffinity(0)),
    }


# --------------------------------------------------------------------------


def measure(name, args, rotations, shared_prefix=False, flushed: int = 0):
    from workloads import make_workload
    t0 = time.perf_counter()
    w = make_workload(name)
    print(f"[bench] {name}: generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
          flush=True)
    st = Stepper(w, rotations, args.splits,
                 w.meta.get("shared_prefix_blocks", 0) if shared_prefix else 0,
                 fused=not args.separate)
    if args.graph and st.fused:
        st.capture()
    ms_step, attn_ms = st.run(args.steps, args.warmup, args.event_every)
    c = alg_counts(w)
    attn_avg = float(np.mean(attn_ms))
    res = dict(w=w, counts=c, ms_step=ms_step, attn_ms_avg=attn_avg, fused=st.fused,
               graph=bool(getattr(st, "graphs", None)),
               attn_ms_p10=float(np.percentile(attn_ms, 10)),
               attn_ms_p50=float(np.percentile(attn_ms, 50)),
               attn_ms_p90=float(np.percentile(attn_ms, 90)))
    print(f"[bench] {name}: {ms_step * 1e3:.1f} us/step, attention {attn_avg * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    if flushed:
        res["flushed_ms"] = st.run_flushed(flushed)
        print(f"[bench] {name}: flushed launches median "
              f"{np.median(res['flushed_ms']) * 1e3:.1f} us", file=sys.stderr, flush=True)
    del st
    import torch
    torch.cuda.empty_cache()
    return res


def measure_copy(args, pairs_n: int, num_blocks: int = 20000):
    """pa_copy_blocks on the decode pool's shape (64 KiB blocks): pairs_n
    forks from distinct sources to distinct fresh blocks, on rotated pools."""
    import torch
    import paged_kv_attention_07_amd as pa
    rng = np.random.default_rng(4242)
    pools = [torch.empty((num_blocks, 2, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
             for _ in range(2)]
    for p in pools:
        p.normal_()
    ids = rng.permutation(num_blocks)[:2 * pairs_n]
    pairs = torch.from_numpy(np.stack([ids[:pairs_n], ids[pairs_n:]], 1).astype(np.int32)).cuda()
    for i in range(args.warmup):
        pa.pa_copy_blocks(pools[i % 2], pairs)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        pa.pa_copy_blocks(pools[i % 2], pairs)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    block_bytes = 2 * 16 * 8 * 128 * 2
    moved = 2 * pairs_n * block_bytes  # read src + write dst
    print(f"[bench] copy_blocks {pairs_n} pairs: {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    del pools
    torch.cuda.empty_cache()
    return {"pairs": pairs_n, "block_bytes": block_bytes, "avg_us": round(ms * 1e3, 2),
            "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
            "pct_peak_hbm": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


def measure_serve(name: str = "serve_llama3_2k"):
    """The multi-step driver over a synthetic serving trace: the C++
    scheduler plans every step (prefix hits, chunked prefill, forks), one
    metadata copy, block copies, slot mapping, K/V scatter and attention on
    the GPU.  One attention layer per step (no model): tokens/s here is the
    rate at which the engine turns scheduled tokens into attention output."""
    import torch
    from paged_kv_attention_07_amd.engine import Engine
    from workloads.trace import step_inputs, trace
    t = trace(name)
    Hq, Hkv, D = 32, 8, 128
    q, k, v = step_inputs(t.seed, 0, t.max_num_batched_tokens, Hq, Hkv, D, "bf16")
    dev = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (q, k, v)]
    # sampled tokens, looked up per (request, step): the stand-in for a model
    max_id = max([r for a in t.arrivals.values() for r, _, _ in a] +
                 [c for f in t.forks.values() for _, c, _ in f]) + 1
    table = np.array([[t.sampled(r, st) for st in range(t.num_steps)] for r in range(max_id)],
                     dtype=np.int32)

    def run():
        eng = Engine(num_blocks=t.num_blocks, max_num_batched_tokens=t.max_num_batched_tokens,
                     max_num_seqs=t.max_num_seqs, max_model_len=t.max_model_len, num_q_heads=Hq,
                     num_kv_heads=Hkv, head_dim=D, dtype="bf16")
        host_s, tokens, steps, gpu_ms = 0.0, 0, 0, []
        # events around every tenth step only: each record costs host time,
        # which this host-and-GPU loop would otherwise pay on every step
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  if i % 10 == 0 else None for i in range(t.num_steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for step in range(t.num_steps):
            for rid, prompt, n in t.arrivals.get(step, []):
                eng.add_request(rid, prompt, n)
            for parent, child, n in t.forks.get(step, []):
                eng.fork(parent, child, n)
            h0 = time.perf_counter()
            ev = events[steps]
            if ev:
                ev[0].record()
            st = eng.step(*dev)
            if ev:
                ev[1].record()
            if st.num_seqs == 0:
                eng.update([])
                if not eng.stats()["num_waiting"] and step > max(t.arrivals):
                    break
                continue
            eng.update(table[st.request_ids, step])
            host_s += time.perf_counter() - h0
            tokens += st.num_tokens
            steps += 1

        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms.extend(ev[0].elapsed_time(ev[1]) for ev in events[:steps] if ev)
        stats = eng.stats()
        eng.close()
        del eng
        torch.cuda.empty_cache()
        return wall, host_s, tokens, steps, stats, float(np.mean(gpu_ms))

    run()                                   # warm-up pass over the same trace
    wall, host_s, tokens, steps, stats, gpu_step_ms = run()
    print(f"[bench] serve {name}: {steps} steps, {tokens} tokens in {wall * 1e3:.1f} ms",
          file=sys.stderr, flush=True)
    return {"trace": name, "steps": steps, "tokens": tokens,
            "tokens_per_s": round(tokens / wall, 1), "ms_per_step": round(wall * 1e3 / steps, 4),
            "host_us_per_step": round(host_s * 1e6 / steps, 1),
            "gpu_us_per_step": round(gpu_step_ms * 1e3, 1),
            "prefix_hit_tokens": stats["total_prefix_hit_tokens"],
            "preemptions": stats["total_preemptions"],
            "layer": "Llama-3-8B attention layer (Hq 32, Hkv 8, D 128, bf16)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (one-launch steps only)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="bracket every N-th timed step's attention call with HIP events "
                         "(1: every step)")
    ap.add_argument("--separate", action="store_true",
                    help="slot mapping, reshape_and_cache and attention as three calls "
                         "(default: one cache-and-attend launch)")
    ap.add_argument("--extra", action="store_true", help="also time the prefix-shared and "
                    "long-context decode batches")
    ap.add_argument("--only", choices=sorted(WORKLOADS) + ["copy", "serve"], default=None)
    ap.add_argument("--flushed", type=int, default=60,
                    help="cold-cache launches of the headline leg, each after a 512 MiB "
                         "flush (0: skip)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy 1 GiB device-to-device 3 times (a kernel of "
                         "known traffic, to calibrate the profiler's FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rot = 4
    names = [args.only] if args.only else ["decode", "mixed", "chunk"] + (
        ["prefix", "prefixplain", "long", "prefill2k", "prefill8k", "prefillbatch"]
        if args.extra else [])
    copy_lines, serve_line = [], None
    if args.only == "copy" or (args.extra and not args.only):
        copy_lines = [measure_copy(args, n) for n in (16, 256, 4096)]
    if args.only == "serve" or (args.extra and not args.only):
        serve_line = measure_serve()
    if args.only in ("copy", "serve"):
        names = ["decode"]
    names = [n for n in names if n in WORKLOADS]
    # the prefix-shared batch runs the shared-prefix decode ("prefix") and the
    # plain decode ("prefixplain") on the same inputs
    results = {k: measure(WORKLOADS[k], args, rot if k != "long" else 2,
                          shared_prefix=(k == "prefix"),
                          flushed=args.flushed if k == names[0] else 0) for k in names}

    # the headline is the decode batch; with --only <leg> it is that leg, with
    # the roofline of the kernel that dominates it
    head_key = "decode" if "decode" in results else next(iter(results))
    head = results[head_key]
    w, c = head["w"], head["counts"]
    attn_bytes = c["attn_unique"] if head_key in ("prefix", "prefixplain") else c["attn_logical"]
    step_bytes = attn_bytes + c["scatter"] + c["slots"]
    value = step_bytes / (head["ms_step"] * 1e-3) / 1e9
    achieved = c["attn_logical"] / (head["attn_ms_avg"] * 1e-3) / 1e9
    launch = {"avg_launch_us": round(head["attn_ms_avg"] * 1e3, 2),
              "p10_us": round(head["attn_ms_p10"] * 1e3, 2),
              "p50_us": round(head["attn_ms_p50"] * 1e3, 2),
              "p90_us": round(head["attn_ms_p90"] * 1e3, 2)}
    if head_key in ("chunk", "prefill2k", "prefill8k", "prefillbatch"):
        tflops = c["chunk_flops"] / (head["attn_ms_avg"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tflops, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": ("pa_cache_and_attend_mixed" if head["fused"]
                               else "pa_attention_mixed") + " (prefill_tile_kernel)",
                    "alg_flops_per_launch": int(c["chunk_flops"]), **launch}
    else:
        # shared-prefix batches are priced on unique bytes (the prefix once)
        alg = c["attn_unique"] if head_key in ("prefix", "prefixplain") else c["attn_logical"]
        if head["fused"]:
            # the launch also reads the new K/V rows, stores them and the slots
            alg += c["scatter"] + 8 * w.num_tokens
        achieved = alg / (head["attn_ms_avg"] * 1e-3) / 1e9
        dec = "pa_cache_and_attend_decode" if head["fused"] else "pa_attention_decode"
        kernel = {"decode": dec + " (decode_split_kernel + decode_merge_kernel)",
                  "prefix": "pa_attention_decode_shared_prefix",
                  "prefixplain": dec, "long": dec,
                  "mixed": "pa_cache_and_attend_mixed" if head["fused"]
                  else "pa_attention_mixed"}.get(head_key, head_key)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic("decode_split_kernel")
                    if head_key == "decode" else None,
                    "traffic_kernel": "decode_split_kernel (profiles/traffic.json)",
                    "kernel": kernel, "alg_bytes_per_launch": int(alg), **launch}
    if head.get("flushed_ms"):
        fm = np.asarray(head["flushed_ms"])
        alg_bytes = roofline.get("alg_bytes_per_launch")
        roofline["flushed"] = {
            "method": "before each launch a 512 MiB write, then a 512 MiB read of another "
                      "buffer, evict L2 and the Infinity Cache; HIP events around the "
                      "attention call alone",
            "launches": int(fm.size),
            "median_us": round(float(np.median(fm)) * 1e3, 2),
            "p10_us": round(float(np.percentile(fm, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(fm, 90)) * 1e3, 2),
            "achieved_at_median": (round(alg_bytes / (float(np.median(fm)) * 1e-3) / 1e9, 1)
                                   if alg_bytes else None)}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": DESCR.get(w.name, ""),
                   "num_seqs": w.num_seqs, "query_tokens": w.num_tokens,
                   "keys": int(w.seq_lens.sum()), "pool_blocks": w.num_blocks,
                   "step": ("slot_mapping + reshape_and_cache + attention in one launch "
                            "(pa_cache_and_attend_*) + split merge" if head["fused"] else
                            "slot_mapping + reshape_and_cache + attention (three calls)"),
                   "pool_rotation": rot, "num_splits": args.splits or "auto"},
        "pct_peak_hbm": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "gpu": gpu_info(),
        "hbm_reference": copy_reference(),
    }
    if "mixed" in results:
        m = results["mixed"]
        mw, mc = m["w"], m["counts"]
        mbytes = mc["attn_logical"] + mc["scatter"] + mc["slots"]
        line["mixed_step"] = {
            "workload": mw.name, "tokens_per_s": round(mw.num_tokens / (m["ms_step"] * 1e-3), 1),
            "ms_per_step": round(m["ms_step"], 5), "query_tokens": mw.num_tokens,
            "hbm_gbs": round(mbytes / (m["ms_step"] * 1e-3) / 1e9, 1),
            "pct_peak_hbm": round(100 * mbytes / (m["ms_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "attention_avg_us": round(m["attn_ms_avg"] * 1e3, 2),
            "chunk_gflop": round(mc["chunk_flops"] / 1e9, 3),
        }
    if "chunk" in results:
        ch = results["chunk"]
        cw, cc = ch["w"], ch["counts"]
        tflops = cc["chunk_flops"] / (ch["attn_ms_avg"] * 1e-3) / 1e12
        line["prefill_chunk"] = {
            "workload": cw.name, "attention_avg_us": round(ch["attn_ms_avg"] * 1e3, 2),
            "gflop": round(cc["chunk_flops"] / 1e9, 3), "tflops": round(tflops, 1),
            "mfma_util": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(cw.num_tokens / (ch["ms_step"] * 1e-3), 1),
        }
    for key in ("prefill2k", "prefill8k", "prefillbatch"):
        if key in results:
            r = results[key]
            rw, rc = r["w"], r["counts"]
            tf = rc["chunk_flops"] / (r["attn_ms_avg"] * 1e-3) / 1e12
            line[key] = {
                "workload": rw.name, "attention_avg_us": round(r["attn_ms_avg"] * 1e3, 2),
                "gflop": round(rc["chunk_flops"] / 1e9, 2), "tflops": round(tf, 1),
                "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "tokens_per_s": round(rw.num_tokens / (r["ms_step"] * 1e-3), 1),
            }
    for key in ("prefix", "prefixplain", "long"):
        if key in results:
            r = results[key]
            rw, rc = r["w"], r["counts"]
            line[f"{key}_decode"] = {
                "entry": ("pa_attention_decode_shared_prefix" if key == "prefix"
                          else "pa_cache_and_attend_decode" if r["fused"]
                          else "pa_attention_decode"),
                "workload": rw.name,
                "attention_avg_us": round(r["attn_ms_avg"] * 1e3, 2),
                "hbm_gbs_unique": round(rc["attn_unique"] / (r["attn_ms_avg"] * 1e-3) / 1e9, 1),
                "effective_gbs_logical": round(rc["attn_logical"] / (r["attn_ms_avg"] * 1e-3) / 1e9, 1),
                "ms_per_step": round(r["ms_step"], 5),
            }
    if copy_lines:
        line["copy_blocks"] = copy_lines
    if serve_line:
        line["serve"] = serve_line
    if args.copy_probe:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = 1 << 30
        del src, dst
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
