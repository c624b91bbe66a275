"""Benchmark of the paged-KV-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--extra] [--only LEG] [--splits S] [--separate] [--graph]

A step is one pass of the whole path over one batch: slot mapping of the new
tokens, reshape_and_cache of their K/V, then attention (decode for the decode
batches, mixed for the chunked-prefill batch).  By default the three run as
one attention launch (pa_cache_and_attend_*: the launch stores the new tokens
and reads them from the input rows) plus the split merge; --separate times
the three calls one after the other.  Inputs are resident in HBM before
timing starts; several copies of the KV pool are rotated so that successive
steps do not hit in the 256 MB Infinity Cache.

Legs of a plain run, one per workload of the five configurations:
  decode  64-request Llama-3-8B-layer decode batch (the headline `value`)
  mixed   chunked-prefill mixed step (593 query tokens)
  chunk   that step's 512-token prefill chunk alone (matrix-core utilisation)
  prefix  256-request decode sharing a 1024-token prefix (priced on unique bytes)
  long    16 x 32768-token decode (split-KV partition-and-reduce)
  tiny    the tiny fp32 decode (launch-bound: microseconds only)
--extra adds the long-prefill legs, the prefix batch through plain decode,
pa_copy_blocks and the serving-trace engine.

Each leg times K steps back to back.  `ms_per_step` is host wall time; the
GPU time per step comes from one pair of HIP events recorded on the launch
stream around the same K steps, and every leg's `roofline` divides the
step's algorithmic bytes (or flops) by it.  The CPU oracle is timed on the
headline batch over all host cores, before the GPU is first touched.
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
    "chunk": "prefill_chunk_bf16",
    "prefix": "prefix_shared_decode_bf16",
    "long": "long_context_decode_bf16",
    "tiny": "tiny_f32_decode",
    "prefixplain": "prefix_shared_decode_bf16",
    "prefill2k": "prefill_chunk_2048_bf16",
    "prefill8k": "prefill_8192_bf16",
    "prefillbatch": "prefill_batch_4x1024_bf16",
}
DEFAULT_LEGS = ["decode", "mixed", "chunk", "prefix", "long", "tiny"]
EXTRA_LEGS = ["prefixplain", "prefill2k", "prefill8k", "prefillbatch"]
MFMA_LEGS = {"chunk", "prefill2k", "prefill8k", "prefillbatch"}
UNIQUE_LEGS = {"prefix", "prefixplain"}    # priced on unique bytes (shared prefix once)

DESCR = {
    "decode_bf16_64req": "Llama-3-8B layer decode (Hq 32, Hkv 8, D 128, bf16, block 16): 64 requests, "
                         "seq_len ~ U[512,4096], pool 20000 blocks, 1 new token each",
    "mixed_chunked_prefill_bf16": "Llama-3-8B layer chunked-prefill step: 512-token chunk on 1024 cached, "
                                  "2 x 10-token prefills, 61 decodes at 2048 (593 query tokens)",
    "prefix_shared_decode_bf16": "Llama-3-8B layer decode, 256 requests sharing a 1024-token prefix "
                                 "(64 blocks) + private suffix U[64,512]",
    "long_context_decode_bf16": "Llama-3-8B layer decode, 16 requests at 32768 tokens, pool 36000 blocks",
    "tiny_f32_decode": "fp32 decode, Hq 4, Hkv 2, D 64, 4 requests with seq_lens {5,16,17,100}, "
                       "64-block pool",
    "prefill_chunk_bf16": "Llama-3-8B layer prefill chunk alone: 512 new tokens on 1024 cached",
    "prefill_chunk_2048_bf16": "Llama-3-8B layer prefill: 2048 new tokens on 2048 cached",
    "prefill_8192_bf16": "Llama-3-8B layer prefill: fresh 8192-token prompt",
    "prefill_batch_4x1024_bf16": "Llama-3-8B layer prefill: 4 requests x ~1024-token chunks",
}


# --------------------------------------------------------------------------
# algorithmic byte / flop counts (what the method itself must move)
# --------------------------------------------------------------------------


def alg_counts(w, fused: bool = True):
    """Bytes one step must move, and the attention's flops.

    attention: K/V of every visible key (logical: per request; unique: each
    physical slot once), q in and out, one table entry per block read and
    three int32 of metadata per request.  step: attention plus the new
    tokens' K/V read from the input and stored into the cache, and their
    slots written (the one-launch step returns them).  In the one-launch
    step (`fused`) the attention takes the new tokens' keys and values from
    the input rows it reads anyway, so their cache reads are not counted;
    the three-call step stores them first and reads them back."""
    esz = 4 if w.dtype == "f32" else 2
    Hq, Hkv, D, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    T, R = w.num_tokens, w.num_seqs
    kb = 2 * Hkv * D * esz                       # K+V bytes per token per layer
    ql = w.q_lens
    rows = ql > 0
    keys_read = int(w.seq_lens[rows].astype(np.int64).sum())
    used_tokens = 0
    seen = set()
    for r in np.nonzero(rows)[0]:
        L = int(w.seq_lens[r])
        for j in range(-(-L // B)):
            blk = int(w.block_table[r, j])
            if blk in seen:
                continue
            seen.add(blk)
            used_tokens += min(B, L - j * B)
    nblocks = int(sum(-(-int(L) // B) for L in w.seq_lens[rows]))
    qo = 2 * T * Hq * D * esz
    meta = nblocks * 4 + R * 4 * 3
    attn_logical = keys_read * kb + qo + meta
    attn_unique = used_tokens * kb + qo + meta
    new_rows = 2 * T * kb + 8 * T
    pairs = chunk_pairs = 0
    for r in np.nonzero(rows)[0]:
        c, n = int(w.num_computed[r]), int(ql[r])
        pairs += n * c + n * (n + 1) // 2
        if n > 1:
            chunk_pairs += n * c + n * (n + 1) // 2
    reread = 0 if fused else T * kb               # the new rows read back from the cache
    return dict(attn_logical=attn_logical, attn_unique=attn_unique, new_rows=new_rows,
                step_logical=attn_logical - T * kb + reread + new_rows,
                step_unique=attn_unique - T * kb + reread + new_rows,
                flops=4 * D * Hq * pairs, chunk_flops=4 * D * Hq * chunk_pairs,
                kv_bytes_per_token=kb)


# --------------------------------------------------------------------------
# CPU oracle baseline, all host cores (run before the GPU is touched)
# --------------------------------------------------------------------------

_CPU_STATE = {}


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass


def _cpu_worker(reqs):
    import oracle
    w, pool = _CPU_STATE["w"], _CPU_STATE["pool"]
    out = oracle.paged_attention(w.q, pool, w.block_table, w.seq_lens, w.query_start_loc,
                                 w.num_computed, w.scale, w.dtype, requests=reqs)
    rows = np.concatenate([np.arange(w.query_start_loc[r], w.query_start_loc[r + 1])
                           for r in reqs])
    return out[rows]


def cpu_baseline(w, budget_s: float = 10.0):
    """The oracle as it stands on the whole batch: its scatter (a copy of the
    pool with the new rows stored) once, then its attention with the requests
    dealt over one worker process per host core (BLAS one thread each),
    full passes until about `budget_s` of wall time, best pass kept.
    Returns the step's algorithmic bytes per second, as the GPU figure."""
    import multiprocessing as mp

    import oracle
    cores = len(os.sched_getaffinity(0))
    slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, w.block_size)
    t0 = time.perf_counter()
    pool = oracle.reshape_and_cache(w.pool, w.k_new, w.v_new, slots)
    t_scatter = time.perf_counter() - t0
    order = sorted((r for r in range(w.num_seqs) if w.q_lens[r] > 0),
                   key=lambda r: -int(w.seq_lens[r]) * int(w.q_lens[r]))
    groups = [[] for _ in range(cores)]
    load = [0] * cores
    for r in order:                               # longest first, to the lightest worker
        i = int(np.argmin(load))
        groups[i].append(r)
        load[i] += int(w.seq_lens[r]) * int(w.q_lens[r])
    groups = [g for g in groups if g]
    _CPU_STATE.update(w=w, pool=pool)
    best, spent, passes = float("inf"), 0.0, 0
    try:
        with mp.get_context("fork").Pool(len(groups), initializer=_cpu_worker_init) as p:
            p.map(_cpu_worker, [[g[0]] for g in groups], chunksize=1)   # start-up
            while passes < 3 or (spent < budget_s and passes < 50):
                t0 = time.perf_counter()
                p.map(_cpu_worker, groups, chunksize=1)
                dt = time.perf_counter() - t0
                best, spent, passes = min(best, dt), spent + dt, passes + 1
    finally:
        _CPU_STATE.clear()
    c = alg_counts(w)
    toks = int(sum(int(w.q_lens[r]) for r in order))
    t_total = t_scatter + best
    return {
        "value": round(c["step_logical"] / t_total / 1e9, 4), "unit": "GB/s",
        "cores": len(groups), "kind": "oracle",
        "sample": f"all {len(order)} requests of {w.name} ({toks} query tokens, "
                  f"{int(w.seq_lens.sum())} keys): the oracle's scatter once on one core "
                  f"({t_scatter:.3f} s, a copy of the {w.pool.nbytes / 1e9:.2f} GB pool with "
                  f"the new rows stored) + its fp64 numpy attention with the requests dealt "
                  f"over {len(groups)} worker processes, BLAS 1 thread each, best of {passes} "
                  f"full passes ({best:.3f} s)",
        "scatter_s": round(t_scatter, 4), "attention_s": round(best, 4),
        "tokens_per_s": round(toks / t_total, 3),
        "cpu": platform.processor() or platform.machine(),
        "host_cores_available": cores,
    }


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
        self.fused = fused
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

    def _fused(self, kv):
        pa, w = self.pa, self.w
        if self.decode and self.shared_prefix:
            pa.pa_cache_and_attend_decode_shared_prefix(
                self.q, self.kn, self.vn, kv, self.bt, self.sl, w.scale, w.max_seq_len,
                self.shared_prefix, out=self.out, slot_mapping=self.slots, workspace=self.ws,
                num_splits=self.splits)
        elif self.decode:
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

    def step(self, i, ev=None):
        """One step over pool copy i; with `ev`, HIP events bracket the
        attention call alone."""
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
            self._fused(kv)
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

    def run(self, steps: int, warmup: int):
        """Time `steps` steps back to back.  Returns (host ms per step, GPU ms
        per step): the host figure is wall time between two synchronisations;
        the GPU figure comes from one pair of HIP events recorded on the
        launch stream before the first and after the last timed step, so no
        event sits between two steps (an event pair around each step adds
        ~2 us of event latency per step to what it brackets)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            self.step(warmup + i)
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter passes (profiles/traffic.json), or None when the
    kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[f"{kernel}@{workload}"]
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


def _median_event_ms(fn, reps: int):
    import torch
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.median(ms))


def hbm_references(copy_bytes: int = 1 << 30, read_bytes: int = 4 << 30, reps: int = 10):
    """Achievable-bandwidth references, median of `reps` event-timed runs
    each: a device-to-device copy (torch; read + write counted) and the
    library's streaming read probe (pa_read_probe, include/pa_probe.h) over
    `read_bytes` at 1, 2 and 4 wavefronts per SIMD."""
    import torch
    import paged_kv_attention_07_amd as pa
    src = torch.ones(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t_copy = _median_event_ms(lambda: dst.copy_(src), reps) * 1e-3
    del src, dst
    x = torch.ones(read_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probe = {}
    for wps in (1, 2, 4):
        pa.pa_read_probe(x, sink, wps)
        torch.cuda.synchronize()
        t = _median_event_ms(lambda: pa.pa_read_probe(x, sink, wps), reps) * 1e-3
        probe[f"{wps}_waves_per_simd"] = round(read_bytes / t / 1e9, 1)
    del x, sink
    torch.cuda.empty_cache()
    cgbs = 2 * copy_bytes / t_copy / 1e9
    best = max(probe.values())
    return {
        "copy": {"kind": "device-to-device copy (torch), read + write bytes / median time",
                 "bytes": 2 * copy_bytes, "gbs": round(cgbs, 1),
                 "pct_peak_hbm": round(100 * cgbs / HBM_PEAK_GBS, 2)},
        "read": {"kind": "streaming read (pa_read_probe), bytes read / median time; best "
                         "of the wave counts",
                 "bytes": read_bytes, "gbs": best, "by_waves_per_simd": probe,
                 "pct_peak_hbm": round(100 * best / HBM_PEAK_GBS, 2)},
    }


# --------------------------------------------------------------------------
# legs
# --------------------------------------------------------------------------


def _entry(key, fused):
    if key == "prefix":
        return ("pa_cache_and_attend_decode_shared_prefix" if fused else
                "pa_attention_decode_shared_prefix (three calls)")
    if key in ("decode", "long", "tiny", "prefixplain"):
        return "pa_cache_and_attend_decode" if fused else "pa_attention_decode (three calls)"
    return "pa_cache_and_attend_mixed" if fused else "pa_attention_mixed (three calls)"


DOMINANT = {
    "decode": "decode_split_kernel", "long": "decode_split_kernel",
    "prefixplain": "decode_split_kernel", "tiny": "decode_split_kernel",
    "mixed": "fused_attention_kernel", "prefix": "fused_attention_kernel",
    "chunk": "prefill_tile_kernel", "prefill2k": "prefill_tile_kernel",
    "prefill8k": "prefill_tile_kernel", "prefillbatch": "fused_attention_kernel",
}


def measure(key, args, w=None, flushed: int = 0):
    import torch
    from workloads import make_workload
    name = WORKLOADS[key]
    if w is None:
        t0 = time.perf_counter()
        w = make_workload(name)
        print(f"[bench] {name}: generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
              flush=True)
    rotations = 1 if key == "tiny" else 4
    sp = w.meta.get("shared_prefix_blocks", 0) if key == "prefix" else 0
    st = Stepper(w, rotations, args.splits, sp, fused=not args.separate)
    if args.graph and st.fused:
        st.capture()
    ms_step, gpu_ms = st.run(args.steps, args.warmup)
    c = alg_counts(w, fused=st.fused)
    print(f"[bench] {key} ({name}): {ms_step * 1e3:.1f} us/step host, {gpu_ms * 1e3:.1f} us/step "
          f"GPU", file=sys.stderr, flush=True)
    res = dict(key=key, w=w, counts=c, ms_step=ms_step, gpu_ms=gpu_ms, fused=st.fused,
               graph=bool(getattr(st, "graphs", None)), rotations=rotations)
    if flushed:
        res["flushed_ms"] = st.run_flushed(flushed)
        print(f"[bench] {key}: flushed launches median "
              f"{np.median(res['flushed_ms']) * 1e3:.1f} us", file=sys.stderr, flush=True)
    del st
    torch.cuda.empty_cache()
    return res


def leg_line(r):
    """JSON record of one leg: step times and the roofline of its step."""
    key, w, c = r["key"], r["w"], r["counts"]
    gpu_s = r["gpu_ms"] * 1e-3
    line = {"workload": w.name, "description": DESCR.get(w.name, ""),
            "entry": _entry(key, r["fused"]), "graph_replay": r["graph"],
            "ms_per_step": round(r["ms_step"], 5), "gpu_us_per_step": round(r["gpu_ms"] * 1e3, 2),
            "query_tokens": w.num_tokens, "num_seqs": w.num_seqs,
            "tokens_per_s": round(w.num_tokens / (r["ms_step"] * 1e-3), 1)}
    if key == "tiny":
        line["roofline"] = None
        line["note"] = "launch-bound (a 1 MiB pool): microseconds only"
        return line
    unique = key in UNIQUE_LEGS
    alg = c["step_unique"] if unique else c["step_logical"]
    traffic = recorded_traffic(DOMINANT[key], w.name) if r["fused"] else None
    if key in MFMA_LEGS:
        tf = c["chunk_flops"] / gpu_s / 1e12
        line["roofline"] = {
            "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic, "kernel": DOMINANT[key],
            "alg_flops_per_launch": int(c["chunk_flops"]), "alg_bytes_per_launch": int(alg)}
    else:
        gbs = alg / gpu_s / 1e9
        line["roofline"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": DOMINANT[key],
            "alg_bytes_per_launch": int(alg)}
    if traffic:
        line["roofline"]["traffic_over_alg_bytes"] = round(traffic / alg, 4)
    if key in MFMA_LEGS:
        return line
    if unique:
        line["roofline"]["priced_on"] = "unique bytes (the shared prefix once)"
        line["effective_gbs_logical"] = round(c["step_logical"] / gpu_s / 1e9, 1)
    if key == "mixed":
        line["chunk_gflop"] = round(c["chunk_flops"] / 1e9, 3)
        line["chunk_tflops_over_step"] = round(c["chunk_flops"] / gpu_s / 1e12, 1)
    return line


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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        pa.pa_copy_blocks(pools[i % 2], pairs)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
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
        host_s, tokens, steps = 0.0, 0, 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for step in range(t.num_steps):
            for rid, prompt, n in t.arrivals.get(step, []):
                eng.add_request(rid, prompt, n)
            for parent, child, n in t.forks.get(step, []):
                eng.fork(parent, child, n)
            h0 = time.perf_counter()
            st = eng.step(*dev)
            if st.num_seqs == 0:
                eng.update([])
                if not eng.stats()["num_waiting"] and step > max(t.arrivals):
                    break
                continue
            eng.update(table[st.request_ids, step])
            host_s += time.perf_counter() - h0
            tokens += st.num_tokens
            steps += 1
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stats = eng.stats()
        eng.close()
        del eng
        torch.cuda.empty_cache()
        return wall, host_s, tokens, steps, stats, e0.elapsed_time(e1)

    run()                                   # warm-up pass over the same trace
    wall, host_s, tokens, steps, stats, gpu_span_ms = run()
    print(f"[bench] serve {name}: {steps} steps, {tokens} tokens in {wall * 1e3:.1f} ms",
          file=sys.stderr, flush=True)
    return {"trace": name, "steps": steps, "tokens": tokens,
            "tokens_per_s": round(tokens / wall, 1), "ms_per_step": round(wall * 1e3 / steps, 4),
            "host_us_per_step": round(host_s * 1e6 / steps, 1),
            "gpu_span_us_per_step": round(gpu_span_ms * 1e3 / steps, 1),
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
    ap.add_argument("--separate", action="store_true",
                    help="slot mapping, reshape_and_cache and attention as three calls "
                         "(default: one cache-and-attend launch)")
    ap.add_argument("--extra", action="store_true",
                    help="also the long-prefill legs, plain decode of the prefix batch, "
                         "pa_copy_blocks and the serving-trace engine")
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

    if args.only in ("copy", "serve"):
        keys = []
    elif args.only:
        keys = [args.only]
    else:
        keys = DEFAULT_LEGS + (EXTRA_LEGS if args.extra else [])

    # the oracle baseline forks one worker per host core: it runs first, on the
    # headline batch, before anything initialises the GPU in this process
    from workloads import make_workload
    head_key = keys[0] if keys else "decode"
    t0 = time.perf_counter()
    head_w = make_workload(WORKLOADS[head_key])
    print(f"[bench] {head_w.name}: generated in {time.perf_counter() - t0:.1f}s",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head_w)
        print(f"[bench] cpu baseline: {cpu['value']} GB/s on {cpu['cores']} cores",
              file=sys.stderr, flush=True)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    results = {}
    for k in keys:
        results[k] = measure(k, args, w=head_w if k == head_key else None,
                             flushed=args.flushed if k == head_key else 0)
    copy_lines, serve_line = [], None
    if args.only == "copy" or (args.extra and not args.only):
        copy_lines = [measure_copy(args, n) for n in (16, 256, 4096)]
    if args.only == "serve" or (args.extra and not args.only):
        serve_line = measure_serve()
    if not results:   # copy / serve alone: the decode leg stays the headline
        results["decode"] = measure("decode", args, w=head_w)
        head_key = "decode"

    legs = {k: leg_line(r) for k, r in results.items()}
    head = results[head_key]
    hw, hc, hl = head["w"], head["counts"], legs[head_key]
    if head_key in MFMA_LEGS or head_key == "tiny":
        value, unit = hl["tokens_per_s"], "tokens/s"
    else:
        step_bytes = hc["step_unique"] if head_key in UNIQUE_LEGS else hc["step_logical"]
        value, unit = step_bytes / (head["ms_step"] * 1e-3) / 1e9, "GB/s"
    roofline = dict(hl["roofline"] or {})
    if roofline:
        roofline["gpu_us_per_step"] = hl["gpu_us_per_step"]
        roofline["timing"] = ("algorithmic bytes (flops) of the step / GPU time per step from "
                              "one pair of HIP events on the launch stream around the "
                              f"{args.steps} timed steps (the step: the attention launch and "
                              "its split merge)")
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
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hw.dtype,
        "data": "synthetic",
        "config": {"workload": hw.name, "description": DESCR.get(hw.name, ""),
                   "num_seqs": hw.num_seqs, "query_tokens": hw.num_tokens,
                   "keys": int(hw.seq_lens.sum()), "pool_blocks": hw.num_blocks,
                   "step": ("slot_mapping + reshape_and_cache + attention in one launch "
                            "(pa_cache_and_attend_*) + split merge" if head["fused"] else
                            "slot_mapping + reshape_and_cache + attention (three calls)"),
                   "pool_rotation": head["rotations"], "num_splits": args.splits or "auto"},
        "pct_peak_hbm": round(100 * value / HBM_PEAK_GBS, 2) if unit == "GB/s" else None,
        "roofline": roofline or None,
        "legs": legs,
    }
    if "mixed" in legs:
        m = legs["mixed"]
        line["mixed_step"] = {"workload": m["workload"], "tokens_per_s": m["tokens_per_s"],
                              "ms_per_step": m["ms_per_step"],
                              "hbm_frac": m["roofline"]["frac"]}
    line["gpu"] = gpu_info()
    line["hbm_reference"] = hbm_references()
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
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
