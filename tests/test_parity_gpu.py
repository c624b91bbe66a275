"""HIP path vs the fp64 oracle on the same seeded inputs, through the C ABI.

Bars: slot mapping and reshape_and_cache bit-exact (whole pool, NaN payloads
included); attention within 1e-5 max-abs for fp32 and within 2e-2 max-abs and
2e-3 mean-abs for bf16/f16.  Slots attention must not read are NaN-poisoned,
and so are the slots this step's tokens are written to, so a read of a stale
or foreign slot shows up as a non-finite output.
"""

import functools
import math

import numpy as np
import pytest

import oracle
from workloads import make_workload
from workloads.gen import build_workload

import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import paged_kv_attention_07_amd as pa  # noqa: E402  (fails loudly if libpa.so is missing)

SMALL = ["tiny_f32_decode", "tiny_f32_decode_alt", "decode_bf16_small", "mixed_bf16_small",
         "prefix_shared_small", "long_decode_small"]


@functools.lru_cache(maxsize=4)
def workload(name, seed=None):
    print(f"[workload] {name} seed={seed}", flush=True)
    return make_workload(name, seed)


def full_check(w, requests=None, **kw):
    print(f"[case] {w.name} seed={w.seed} R={w.num_seqs} T={w.num_tokens} {kw}", flush=True)
    pool, g_slots, g_pool, g_out = gu.run_step(w, **kw)
    r_slots, r_pool, r_out = gu.oracle_step(w, pool, requests=requests)
    assert np.array_equal(g_slots, r_slots), "slot mapping differs"
    assert np.array_equal(gu.bits(g_pool), gu.bits(r_pool)), "pool differs after the scatter"
    rows = None if requests is None else gu.rows_of(w, requests)
    return gu.check_close(w, g_out, r_out, rows=rows, what=w.name)


# --------------------------------------------------------------------------
# slot mapping + scatter
# --------------------------------------------------------------------------


def test_slot_mapping_worked_example():
    """The printed example of the slot formula ("vllm v1 源码精读（三）" §3.4)."""
    bt = gu.ints_to_device(np.array([[5, 12, -1], [3, -1, -1], [7, 21, 9]], np.int32), np.int32)
    sel = gu.ints_to_device(np.array([[5, 12, -1], [7, 21, 9]], np.int32), np.int32)
    qsl = gu.ints_to_device(np.array([0, 1, 2], np.int32), np.int32)
    nc = gu.ints_to_device(np.array([17, 32], np.int32), np.int32)
    got = pa.pa_compute_slot_mapping(sel, qsl, nc, 2, 16).cpu().numpy()
    assert list(got) == [193, 144]
    # a position whose table entry is -1 gets a negative slot
    nc2 = gu.ints_to_device(np.array([0, 16, 40], np.int32), np.int32)
    qsl3 = gu.ints_to_device(np.array([0, 1, 2, 3], np.int32), np.int32)
    got = pa.pa_compute_slot_mapping(bt, qsl3, nc2, 3, 16).cpu().numpy()
    assert got[0] == 5 * 16 and got[1] < 0 and got[2] == 9 * 16 + 8


@pytest.mark.parametrize("name", SMALL)
def test_small_configs(name):
    full_check(workload(name))


def test_reshape_and_cache_padding_and_dtypes():
    """slot < 0 writes nothing; every other byte of the pool is untouched."""
    for dtype, H, D in (("bf16", 8, 128), ("f32", 2, 64), ("f16", 4, 64)):
        w = build_workload(f"rac_{dtype}", dtype=dtype, num_q_heads=H, num_kv_heads=H, head_dim=D,
                           num_blocks=40, requests=[(3, 5), (20, 1), (0, 17)], seed=5,
                           fill_unused="zero")
        dev = gu.Device(w)
        slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, 16)
        slots[[1, 7, 20]] = -1
        dev.scatter(gu.ints_to_device(slots, np.int64))
        want = oracle.reshape_and_cache(w.pool, w.k_new, w.v_new, slots)
        got = gu.from_device(dev.kv, dtype)
        assert np.array_equal(gu.bits(got), gu.bits(want)), dtype


# --------------------------------------------------------------------------
# decode: splits, determinism, invariances, head groupings, dtypes
# --------------------------------------------------------------------------


@pytest.mark.parametrize("splits", [1, 2, 3, 17, 64, 333, 2000])
def test_decode_any_split_count(splits):
    full_check(workload("decode_bf16_small"), num_splits=splits)


def test_decode_deterministic_and_mixed_entry_agrees():
    w = workload("long_decode_small")
    dev = gu.Device(w, gu.poisoned_pool(w))
    dev.scatter(dev.slot_mapping())
    a = gu.from_device(dev.attend(), w.dtype)
    b = gu.from_device(dev.attend(), w.dtype)
    c = gu.from_device(dev.attend(force_mixed=True), w.dtype)
    assert np.array_equal(a, b), "two identical launches differ"
    assert np.array_equal(a, c), "decode rows through the mixed entry differ"


def test_decode_block_permutation_bit_identical():
    """Relabelling physical blocks leaves the GPU result bit-identical."""
    w = workload("decode_bf16_small")
    pool = gu.poisoned_pool(w)
    _, _, _, out1 = gu.run_step(w, poison=True)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    import dataclasses
    w2 = dataclasses.replace(w, pool=pool2, block_table=bt2)
    dev = gu.Device(w2, pool2)
    dev.scatter(dev.slot_mapping())
    out2 = gu.from_device(dev.attend(), w.dtype)
    assert np.array_equal(out1, out2)


def test_prefix_sharing_bit_identical_to_private_copies():
    w = workload("prefix_shared_small")
    pool = gu.poisoned_pool(w)
    dev = gu.Device(w, pool)
    dev.scatter(dev.slot_mapping())
    shared = gu.from_device(dev.attend(), w.dtype)
    # copy the shared blocks into free blocks, one private copy per request
    S = 4
    free = np.setdiff1d(np.arange(w.num_blocks), w.used_blocks)
    assert free.size >= S * w.num_seqs
    pool2, bt2, k = pool.copy(), w.block_table.copy(), 0
    for r in range(w.num_seqs):
        for j in range(S):
            pool2[free[k]] = pool[w.block_table[r, j]]
            bt2[r, j] = free[k]
            k += 1
    import dataclasses
    w2 = dataclasses.replace(w, block_table=bt2)
    dev2 = gu.Device(w2, pool2)
    dev2.scatter(dev2.slot_mapping())
    private = gu.from_device(dev2.attend(), w.dtype)
    assert np.array_equal(shared, private)


def _variant(dtype, Hq, Hkv, D, lens, seed, q_lens=None):
    reqs = [(L - (1 if q_lens is None else q_lens[i]), 1 if q_lens is None else q_lens[i])
            for i, L in enumerate(lens)]
    return build_workload(f"var_{dtype}_{Hq}x{Hkv}x{D}", dtype=dtype, num_q_heads=Hq,
                          num_kv_heads=Hkv, head_dim=D, num_blocks=300, requests=reqs, seed=seed)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [
    ("bf16", 8, 8, 128), ("bf16", 8, 4, 128), ("bf16", 16, 2, 128), ("bf16", 8, 2, 64),
    ("bf16", 4, 4, 64), ("f16", 16, 4, 128), ("f16", 8, 1, 64), ("f32", 8, 2, 128),
    ("f32", 4, 4, 64), ("f32", 16, 2, 64)])
def test_decode_head_groupings_and_dtypes(dtype, Hq, Hkv, D):
    lens = [1, 15, 16, 17, 33, 250, 600, 1000]
    full_check(_variant(dtype, Hq, Hkv, D, lens, seed=11 + Hq + D))
    full_check(_variant(dtype, Hq, Hkv, D, lens, seed=12 + Hq + D), num_splits=5)


@pytest.mark.parametrize("R", [63, 64, 65, 257, 700])
def test_decode_large_batches(R):
    """Each wave scans the batch 64 requests at a time to find its ranges:
    batches around one window and spanning many windows."""
    rng = np.random.default_rng(R)
    lens = [int(x) for x in rng.integers(1, 120, size=R)]
    w = build_workload(f"many_{R}", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64,
                       num_blocks=sum(-(-L // 16) for L in lens) + 8,
                       requests=[(L - 1, 1) for L in lens], seed=R)
    full_check(w)
    full_check(w, num_splits=37)
    full_check(w, fused=True)


def test_decode_single_key_returns_v0():
    w = _variant("bf16", 8, 2, 128, [1, 1, 1], seed=3)
    pool, _, g_pool, out = gu.run_step(w)
    for r in range(3):
        blk = w.block_table[r, 0]
        v0 = g_pool[blk, 1, 0]                 # [Hkv, D] bits written by the scatter
        for h in range(8):
            assert np.array_equal(out[r, h], v0[h // 4])


# --------------------------------------------------------------------------
# mixed (chunked-prefill) batches
# --------------------------------------------------------------------------


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [
    ("bf16", 32, 8, 128), ("bf16", 8, 8, 128), ("bf16", 8, 4, 64), ("f16", 16, 2, 128),
    ("bf16", 16, 2, 64)])
def test_mixed_groupings(dtype, Hq, Hkv, D):
    lens = [40, 17, 300, 5, 64, 129, 1, 700]
    q_lens = [40, 2, 33, 1, 16, 100, 1, 64]
    full_check(_variant(dtype, Hq, Hkv, D, lens, seed=21 + Hq, q_lens=q_lens))


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (8, 4, 64), (8, 2, 128), (16, 2, 64),
                                      (32, 8, 128)])
def test_mixed_f32(Hq, Hkv, D):
    """fp32 cache: chunks go to the vector-ALU tiles (every head grouping), decode
    rows to the split; chunk lengths 2..100 across tile edges, chunks starting
    mid-block, a request with no tokens this step, 1e-5 vs the oracle."""
    lens = [40, 17, 300, 5, 64, 129, 1, 700, 90, 33]
    q_lens = [40, 2, 33, 1, 16, 100, 1, 64, 0, 17]
    full_check(_variant("f32", Hq, Hkv, D, lens, seed=71 + Hq + D, q_lens=q_lens))
    # one request alone (tiles only), and one with its whole prompt as the chunk
    full_check(_variant("f32", Hq, Hkv, D, [77], seed=72, q_lens=[60]))
    full_check(_variant("f32", Hq, Hkv, D, [257], seed=73, q_lens=[257]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mixed_chunked_equivalence(dtype):
    """A 1000-token prompt prefilled in chunks 254/254/254/238 ("vllm v1 源码精读（三）"
    §4.2) gives, chunk by chunk, the rows of one full prefill (both vs the oracle)."""
    L = 1000
    full = _variant(dtype, 32, 8, 128, [L], seed=31, q_lens=[L])
    pool = gu.poisoned_pool(full)
    _, _, _, out_full = gu.run_step(full, poison=False)
    _, r_pool, r_full = gu.oracle_step(full, full.pool)
    gu.check_close(full, out_full, r_full, what="full prefill")
    done = 0
    import dataclasses
    for n in oracle.chunk_schedule(L, 254):
        w = dataclasses.replace(
            full, q=full.q[done:done + n], k_new=full.k_new[done:done + n],
            v_new=full.v_new[done:done + n], seq_lens=np.array([done + n], np.int32),
            num_computed=np.array([done], np.int32),
            query_start_loc=np.array([0, n], np.int32))
        dev = gu.Device(w, r_pool)  # cache already holds every token's K/V
        out = gu.from_device(dev.attend(force_mixed=True), w.dtype)
        gu.check_close(w, out, r_full[done:done + n], what=f"chunk at {done}")
        done += n


def test_mixed_request_order_shuffled():
    w = workload("mixed_bf16_small")
    rng = np.random.default_rng(5)
    order = rng.permutation(w.num_seqs)
    ql = w.q_lens[order]
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    rows = gu.rows_of(w, order)
    import dataclasses
    w2 = dataclasses.replace(w, q=w.q[rows], k_new=w.k_new[rows], v_new=w.v_new[rows],
                             seq_lens=w.seq_lens[order], num_computed=w.num_computed[order],
                             block_table=w.block_table[order], query_start_loc=qsl)
    full_check(w2)


# --------------------------------------------------------------------------
# full-size configurations, every request against the oracle
# --------------------------------------------------------------------------


def test_full_decode_64req():
    full_check(workload("decode_bf16_64req"))


def test_full_mixed_step():
    full_check(workload("mixed_chunked_prefill_bf16"))


def test_full_prefix_shared():
    """All 256 requests against the oracle (plain decode entry)."""
    full_check(workload("prefix_shared_decode_bf16"))


def test_full_long_context():
    """All 16 requests of 32768 keys against the oracle (~16 s of oracle)."""
    full_check(workload("long_context_decode_bf16"))


CONFIGS = ["tiny_f32_decode", "decode_bf16_64req", "mixed_chunked_prefill_bf16",
           "prefix_shared_decode_bf16", "long_context_decode_bf16"]


@pytest.mark.parametrize("i", range(1, 6))
@pytest.mark.parametrize("seed_base", [2000, 3000])
def test_configs_at_more_seeds(seed_base, i):
    """Configuration i of the five (tiny fp32, 64-request decode, mixed step,
    prefix-shared, long-context) at seeds 2000 + i and 3000 + i: new lengths,
    tables and values of the same shapes and distributions."""
    name = CONFIGS[i - 1]
    w = workload(name, seed_base + i)
    full_check(w)


def test_workspace_reused_across_calls():
    """One workspace serves many calls with different batches and split
    counts: nothing a call leaves in it affects the next call."""
    import torch
    cases = [(workload("decode_bf16_small"), 7), (workload("long_decode_small"), 0),
             (workload("decode_bf16_small"), 333), (workload("mixed_bf16_small"), 5),
             (workload("long_decode_small"), 64), (workload("tiny_f32_decode"), 0),
             # a larger batch after small ones: its counters must still read zero
             (workload("mixed_chunked_prefill_bf16"), 0), (workload("decode_bf16_small"), 0)]
    nbytes = max(pa.pa_attention_workspace_size(w.num_seqs, w.num_tokens, w.num_q_heads,
                                                w.num_kv_heads, w.head_dim, w.max_seq_len,
                                                w.max_query_len, s) for w, s in cases)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for w, splits in cases:
            pool = gu.poisoned_pool(w)
            dev = gu.Device(w, pool)
            dev.scatter(dev.slot_mapping())
            if w.is_decode_only:
                out = pa.pa_attention_decode(dev.q, dev.kv, dev.block_table, dev.seq_lens,
                                             w.scale, w.max_seq_len, workspace=ws,
                                             num_splits=splits)
            else:
                out = pa.pa_attention_mixed(dev.q, dev.kv, dev.block_table, dev.seq_lens,
                                            dev.qsl, dev.num_computed, w.scale,
                                            w.max_query_len, w.max_seq_len, workspace=ws,
                                            num_splits=splits)
            _, _, ref = gu.oracle_step(w, pool)
            gu.check_close(w, gu.from_device(out, w.dtype), ref, what=f"{w.name}/{splits}")


# --------------------------------------------------------------------------
# long prefill chunks and both prefill tile shapes, every row against the
# oracle
# --------------------------------------------------------------------------

_LARGE_REF = {}


def _large_prefill_check(name, shape, sampled):
    w = workload(name)
    pool = gu.poisoned_pool(w)
    dev = gu.Device(w, pool)
    slots = dev.slot_mapping()
    dev.scatter(slots)
    out = gu.from_device(dev.attend(force_mixed=True, plan=dict(tile_shape=shape)), w.dtype)
    g_pool = gu.from_device(dev.kv, w.dtype)
    r_slots = oracle.slot_mapping(w.block_table, w.query_start_loc, w.num_computed, 16)
    assert np.array_equal(slots.cpu().numpy(), r_slots)
    r_pool = oracle.reshape_and_cache(pool, w.k_new, w.v_new, r_slots)
    assert np.array_equal(gu.bits(g_pool), gu.bits(r_pool))
    if not sampled:
        # the oracle's output does not depend on the tile shape: computed once
        if name not in _LARGE_REF:
            _LARGE_REF[name] = oracle.paged_attention(w.q, r_pool, w.block_table, w.seq_lens,
                                                      w.query_start_loc, w.num_computed,
                                                      w.scale, w.dtype)
        gu.check_close(w, out, _LARGE_REF[name], what=f"{name}/shape{shape}")
        return
    rng = np.random.default_rng(17)
    T = w.num_tokens
    edge = [0, 1, 15, 16, 31, 32, 63, 64, T - 1, T - 2, T - 17]
    rows = np.unique(np.concatenate([edge, rng.choice(T, 53, replace=False)]))
    sub = gu.sampled_rows_check(w, out, rows)
    ref = oracle.paged_attention(sub.q, r_pool, sub.block_table, sub.seq_lens,
                                 sub.query_start_loc, sub.num_computed, w.scale, w.dtype)
    gu.check_close(w, out[rows], ref, what=f"{name}/shape{shape}")


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("name", ["prefill_chunk_2048_bf16", "prefill_batch_4x1024_bf16"])
def test_large_prefill(name, shape):
    _large_prefill_check(name, shape, sampled=False)


def test_prefill_8k():
    """The fresh 8192-token prompt: pool bit-exact, every row against the
    oracle (~20 s of fp64 oracle on the host)."""
    _large_prefill_check("prefill_8192_bf16", 1, sampled=False)


def test_prefill_8k_rows_as_own_requests():
    """The same prompt's rows at tile and block edges plus random ones, each
    recomputed by the oracle as its own one-token request at its position:
    the causal bound of every row follows from the row alone."""
    _large_prefill_check("prefill_8192_bf16", 1, sampled=True)


@pytest.mark.parametrize("scale", [0.01, 0.25, 0.5, 1.0, 2.0])
def test_softmax_scales(scale):
    """Softmax scales other than the pages' 1/sqrt(d_k) (0.088 at D = 128):
    nearly uniform weights, and scales large enough that the scores span
    tens of log2 units and the running max moves on most trips.  Decode
    rows, both tile shapes, tiles beside decode rows, f16 tiles and the fp32
    vector-ALU tiles.

    Bound: up to 0.5 the bf16/f16 bound of the other tests.  From 1.0 on one
    key carries most of a row's weight, so the matrix-core tiles' 16-bit
    probabilities (relative rounding 2^-9 each) no longer average out: the
    error approaches 2^-9 * max|V| (~4.5 here) plus the output's own rounding
    (half an ulp of |out|, up to 2^-7 at |out| ~ 4), so max-abs 3e-2 there;
    the mean-abs bound is unchanged.  fp32: the bound grows with the scale
    from 0.25 on (see below).  The error must not grow with the
    scores' size beyond that (a Q pre-multiplied by the scale and rounded to
    16 bits did: 0.08 at scale 1, 0.16 at 2)."""
    import dataclasses
    lens = [40, 17, 300, 5, 64, 129, 1, 700]
    q_lens = [40, 2, 33, 1, 16, 100, 1, 64]
    cases = [(workload("mixed_bf16_small"), None)]
    cases += [(workload("mixed_bf16_small"), dict(tile_shape=sh, tiles_beside_decode=0))
              for sh in (0, 1)]
    cases += [(workload("decode_bf16_small"), None)]
    cases += [(_variant(dt, Hq, Hkv, D, lens, seed=61 + Hq, q_lens=q_lens), None)
              for dt, Hq, Hkv, D in (("f32", 8, 2, 64), ("f16", 16, 2, 64))]
    for base, plan in cases:
        w = dataclasses.replace(base, scale=scale)
        print(f"[case] scale {scale} {w.name} plan={plan}", flush=True)
        pool, g_slots, g_pool, g_out = gu.run_step(w, plan=plan)
        r_slots, r_pool, r_out = gu.oracle_step(w, pool)
        assert np.array_equal(g_slots, r_slots)
        assert np.array_equal(gu.bits(g_pool), gu.bits(r_pool))
        got = oracle.decode_bits(g_out, w.dtype)
        assert np.all(np.isfinite(got))
        err = np.abs(got - r_out)
        tol = gu.TOL[w.dtype]
        if w.dtype == "f32":
            # fp32 throughout: the exponent's rounding grows with the score's
            # size in log2 units, linearly in the scale (the bound of the other
            # tests holds up to ~0.25)
            max_abs = mean_abs = tol["max_abs"] * max(1.0, 4.0 * scale)
        else:
            max_abs = tol["max_abs"] if scale <= 0.5 else 3e-2
            mean_abs = tol["mean_abs"]
        assert err.max() <= max_abs, f"{w.name} scale {scale}: max abs err {err.max():.3g}"
        assert err.mean() <= mean_abs, f"{w.name} scale {scale}: mean abs err {err.mean():.3g}"


@pytest.mark.parametrize("shape", [0, 1])
def test_mixed_all_tile_shapes(shape):
    """Every prefill tile shape on the small mixed batch and on odd groupings
    (tiles launched on their own, so the shape applies)."""
    plan = dict(tile_shape=shape, tiles_beside_decode=0)
    full_check(workload("mixed_bf16_small"), plan=plan)
    lens = [40, 17, 300, 5, 64, 129, 1, 700]
    q_lens = [40, 2, 33, 1, 16, 100, 1, 64]
    for dtype, Hq, Hkv, D in (("bf16", 8, 8, 128), ("f16", 16, 2, 64), ("bf16", 16, 8, 64)):
        full_check(_variant(dtype, Hq, Hkv, D, lens, seed=41 + Hq, q_lens=q_lens), plan=plan)


# --------------------------------------------------------------------------
# block copies (copy-on-write forks)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("dtype,Hkv,D", [("bf16", 8, 128), ("f32", 2, 64), ("f16", 1, 64),
                                         ("f32", 8, 128)])
def test_copy_blocks_bit_exact(dtype, Hkv, D):
    """Random pairs (with skipped -1 rows) on a pool with NaN payloads: the
    copy is bit-exact and touches nothing but the destinations."""
    import torch
    rng = np.random.default_rng(23 + D + Hkv)
    NB = 300
    w = build_workload("copy", dtype=dtype, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                       num_blocks=NB, requests=[(40, 1)], seed=5 + D, table_width=8)
    pool = w.pool.copy()
    ids = rng.permutation(NB)
    src, dst = ids[:70], ids[70:140]
    pairs = np.stack([src, dst], 1).astype(np.int32)
    pairs[[3, 17], 0] = -1
    pairs[[29], 1] = -1
    kv = gu.to_device(pool, dtype)
    pa.pa_copy_blocks(kv, gu.ints_to_device(pairs, np.int32))
    got = gu.from_device(kv, dtype)
    want = oracle.copy_blocks(pool, pairs)
    assert np.array_equal(gu.bits(got), gu.bits(want))
    # empty call is a no-op
    pa.pa_copy_blocks(kv, gu.ints_to_device(np.zeros((0, 2), np.int32), np.int32))
    torch.cuda.synchronize()
    assert np.array_equal(gu.bits(gu.from_device(kv, dtype)), gu.bits(want))


def test_copy_on_write_parallel_sampling():
    """Parallel sampling: n samples share a prompt whose last block is partly
    filled.  Each sample forks the shared block with pa_copy_blocks, writes
    its own next token into its copy, and decodes; every sample matches the
    oracle, and the shared blocks keep their bits."""
    import dataclasses
    n, prompt = 6, 16 * 20 + 9
    base = build_workload("cow", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                          num_blocks=2000, requests=[(prompt, 1)], seed=77, table_width=32)
    nbp = -(-prompt // 16)
    shared = base.block_table[0, :nbp].copy()
    rng = np.random.default_rng(78)
    spare = np.setdiff1d(np.arange(base.num_blocks), shared)
    fork_dst = rng.choice(spare, n, replace=False).astype(np.int32)
    tables = np.full((n, 32), -1, np.int32)
    for smp in range(n):
        tables[smp, :nbp] = shared
        tables[smp, nbp - 1] = fork_dst[smp]
    pairs = np.stack([np.full(n, shared[-1], np.int32), fork_dst], 1)
    rs = np.random.default_rng(79)
    def bf16(shape):
        x = rs.standard_normal(shape).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    w = dataclasses.replace(
        base, block_table=tables, seq_lens=np.full(n, prompt + 1, np.int32),
        num_computed=np.full(n, prompt, np.int32),
        query_start_loc=np.arange(n + 1, dtype=np.int32),
        q=bf16((n, 32, 128)), k_new=bf16((n, 8, 128)), v_new=bf16((n, 8, 128)))
    dev = gu.Device(w, base.pool)
    pa.pa_copy_blocks(dev.kv, gu.ints_to_device(pairs, np.int32))
    slots = dev.slot_mapping()
    dev.scatter(slots)
    out = gu.from_device(dev.attend(), "bf16")
    g_pool = gu.from_device(dev.kv, "bf16")
    r_pool = oracle.copy_blocks(base.pool, pairs)
    r_slots = oracle.slot_mapping(tables, w.query_start_loc, w.num_computed, 16)
    assert np.array_equal(slots.cpu().numpy(), r_slots)
    r_pool = oracle.reshape_and_cache(r_pool, w.k_new, w.v_new, r_slots)
    assert np.array_equal(gu.bits(g_pool), gu.bits(r_pool))
    assert np.array_equal(gu.bits(g_pool[shared]), gu.bits(base.pool[shared]))
    ref = oracle.paged_attention(w.q, r_pool, tables, w.seq_lens, w.query_start_loc,
                                 w.num_computed, w.scale, "bf16")
    gu.check_close(w, out, ref, what="cow samples")


@pytest.mark.parametrize("overlap", [0, -1])
def test_mixed_with_and_without_concurrent_tiles(overlap):
    """The mixed entry runs prefill tiles and decode ranges in one launch by
    default; both schedules give the oracle's rows, including the one-request
    batch (tiles alone)."""
    plan = dict(tiles_beside_decode=overlap)
    full_check(workload("mixed_bf16_small"), plan=plan)
    lens = [300, 40, 129, 2000, 17]
    q_lens = [100, 1, 64, 1, 1]
    full_check(_variant("bf16", 32, 8, 128, lens, seed=91, q_lens=q_lens), plan=plan)
    full_check(_variant("f16", 8, 2, 64, [77], seed=92, q_lens=[60]), plan=plan)


# --------------------------------------------------------------------------
# decode with a shared prompt prefix read once (cascade)
# --------------------------------------------------------------------------


def test_shared_prefix_small_config():
    w = workload("prefix_shared_small")
    full_check(w, shared_prefix=w.meta["shared_prefix_blocks"])


_PREFIX_REF = {}


@pytest.mark.parametrize("splits", [0, 1, 3, 40])
def test_shared_prefix_full_config(splits):
    """The 256-request batch with a 64-block shared prefix through the
    shared-prefix entry, every request compared with the oracle (the oracle's
    result, the same for every split count, is computed once)."""
    w = workload("prefix_shared_decode_bf16")
    pool, g_slots, g_pool, out = gu.run_step(w, shared_prefix=w.meta["shared_prefix_blocks"],
                                             num_splits=splits)
    if "ref" not in _PREFIX_REF:
        _PREFIX_REF["ref"] = gu.oracle_step(w, pool)
    r_slots, r_pool, ref = _PREFIX_REF["ref"]
    assert np.array_equal(g_slots, r_slots)
    assert np.array_equal(gu.bits(g_pool), gu.bits(r_pool))
    gu.check_close(w, out, ref, what="shared prefix")


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("bf16", 8, 8, 128),
                                            ("f16", 16, 2, 64), ("bf16", 8, 2, 64)])
def test_shared_prefix_edges(dtype, Hq, Hkv, D):
    """Suffixes of every kind after a 5-block prefix: empty (the context is
    exactly the prefix), one key, a partial last block, long; plus the
    prefix-free fallback (P = 0), all against the oracle."""
    P = 5
    lens = [P * 16, P * 16 + 1, P * 16 + 7, P * 16 + 16, P * 16 + 300, P * 16 + 33, 2000]
    w = build_workload(f"sp_{dtype}_{Hq}x{Hkv}x{D}", dtype=dtype, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, num_blocks=600,
                       requests=[(L - 1, 1) for L in lens], seed=61 + Hq + D,
                       shared_prefix_blocks=P)
    full_check(w, shared_prefix=P)
    full_check(w, shared_prefix=0)
    full_check(w, shared_prefix=P, num_splits=2)


@pytest.mark.parametrize("name,P", [("prefix_shared_small", 4), ("sp_edges", 5)])
def test_shared_prefix_matches_plain_decode(name, P):
    """Both decode entries on the same batch agree to a few bf16 ulps of the
    output (each is a bf16-rounded evaluation of the same softmax).  This
    catches keys past the prefix leaking into the prefix pass (rows there
    sit after the keys they may see), which stays near the oracle tolerance
    but is several times the rounding."""
    if name == "sp_edges":
        lens = [P * 16, P * 16 + 1, P * 16 + 7, P * 16 + 16, P * 16 + 300, P * 16 + 33, 2000]
        w = build_workload("sp_edges", dtype="bf16", num_q_heads=8, num_kv_heads=8, head_dim=128,
                           num_blocks=600, requests=[(L - 1, 1) for L in lens], seed=197,
                           shared_prefix_blocks=P)
    else:
        w = workload(name)
    dev = gu.Device(w, gu.poisoned_pool(w))
    dev.scatter(dev.slot_mapping())
    a = oracle.decode_bits(gu.from_device(dev.attend(), w.dtype), w.dtype)
    b = oracle.decode_bits(gu.from_device(dev.attend(shared_prefix=P), w.dtype), w.dtype)
    assert np.max(np.abs(a - b)) <= 6e-3


@pytest.mark.parametrize("name", ["decode_bf16_small", "mixed_bf16_small", "tiny_f32_decode"])
def test_short_names_match_full_names(name):
    """The short-name wrappers (host bounds read back from the device) give the
    bits of the pa_* calls given the same bounds, and the oracle's result."""
    w = workload(name)
    print(f"[case] short names {name}", flush=True)
    pool = gu.poisoned_pool(w)
    outs = []
    for short in (False, True):
        dev = gu.Device(w, pool)
        if short:
            slots = pa.compute_slot_mapping(dev.block_table, dev.qsl, dev.num_computed,
                                            w.num_tokens)
            pa.reshape_and_cache(dev.k_new, dev.v_new, dev.kv, slots)
        else:
            slots = pa.pa_compute_slot_mapping(dev.block_table, dev.qsl, dev.num_computed,
                                               w.num_tokens)
            pa.pa_reshape_and_cache(dev.k_new, dev.v_new, dev.kv, slots)
        args = (dev.q, dev.kv, dev.block_table, dev.seq_lens)
        if w.is_decode_only:
            out = (pa.attention_decode(*args, w.scale) if short else
                   pa.pa_attention_decode(*args, w.scale, w.max_seq_len))
        else:
            args += (dev.qsl, dev.num_computed)
            out = (pa.attention_mixed(*args, w.scale) if short else
                   pa.pa_attention_mixed(*args, w.scale, w.max_query_len, w.max_seq_len))
        outs.append(gu.from_device(out, w.dtype))
    assert np.array_equal(gu.bits(outs[0]), gu.bits(outs[1]))
    _, _, r_out = gu.oracle_step(w, pool)
    gu.check_close(w, outs[1], r_out, what=f"{name} short names")
