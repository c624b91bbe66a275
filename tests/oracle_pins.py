"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` raises AssertionError on failure.  They are called by
test_oracle_pins.py, and test_oracle_mutations.py plants plausible mistakes in
the oracle and requires that at least one of them fails.  Sources are cited by
page title and section:
  [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成"
  [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
  [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"
"""

from __future__ import annotations

import math
import os

import numpy as np

import oracle
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# --------------------------------------------------------------------------
# printed worked examples and closed forms
# --------------------------------------------------------------------------


def check_slot_worked_example():
    """[P4] §3.4: req 0 pos 17 -> slot 193, req 2 pos 32 -> slot 144."""
    rows, cases, B = [], [], None
    for tok in _golden_lines("slot_mapping_worked_example.txt"):
        if tok[0] == "block_size":
            B = int(tok[1])
        elif tok[0] == "block_table_row":
            rows.append([int(x) for x in tok[1:]])
        elif tok[0] == "slot":
            cases.append(tuple(int(x) for x in tok[1:]))
    bt = np.array(rows, dtype=np.int32)
    assert cases
    for r, pos, want in cases:
        assert oracle.slot_of(bt, r, pos, B) == want, (r, pos, want)
    # the same slots through the batched slot_mapping of a one-token step each
    qsl = np.arange(len(cases) + 1, dtype=np.int32)
    bt_sel = bt[[c[0] for c in cases]]
    nc = np.array([c[1] for c in cases], dtype=np.int32)
    got = oracle.slot_mapping(bt_sel, qsl, nc, B)
    assert list(got) == [c[2] for c in cases]


def check_pool_example_shapes():
    """[P4] §3.3: kv_cache[42, 0] is [16, 8, 128]; kv_cache[42, 0, 3] is [8, 128]."""
    for tok in _golden_lines("slot_mapping_worked_example.txt"):
        if tok[0] == "pool_example":
            NB, B, H, D, blk, off = map(int, tok[1:])
    pool = np.zeros((NB, 2, B, H, D), dtype=np.uint16)
    assert pool[blk, 0].shape == (B, H, D)
    assert pool[blk, 0, off].shape == (H, D)
    assert pool.strides[0] == oracle.block_bytes(B, H, D, 2)


def check_size_closed_forms():
    """[P4] §3.1, [P2] §3.1 / §3.3, [P1] §4.2, [P4] §4.2 printed values."""
    n = 0
    for tok in _golden_lines("kv_size_closed_forms.txt"):
        kind, args = tok[0], [int(x) for x in tok[1:]]
        if kind == "kv_bytes_per_token":
            assert oracle.kv_bytes_per_token(*args[:4]) == args[4], tok
        elif kind == "block_bytes":
            assert oracle.block_bytes(*args[:5]) == args[5], tok
        elif kind == "blocks_for_tokens":
            assert oracle.blocks_for_tokens(*args[:2]) == args[2], tok
        elif kind == "chunk_schedule":
            assert oracle.chunk_schedule(*args[:2]) == args[2:], tok
        n += 1
    assert n >= 6


# --------------------------------------------------------------------------
# small random paged problems
# --------------------------------------------------------------------------


def random_paged_problem(rng, *, R=3, Hq=4, Hkv=2, D=8, B=4, NB=40, max_len=20,
                         prefill=False):
    """Per-request contiguous K/V, laid into a pool through a random table.

    Returns (contig, problem) where contig[r] = (Kc [L,Hkv,D], Vc) float32 and
    problem is a dict of oracle arguments (f32 storage)."""
    lens = rng.integers(1, max_len, size=R, endpoint=True)
    nb = [-(-int(L) // B) for L in lens]
    perm = rng.permutation(NB)
    assert sum(nb) <= NB
    bt = np.full((R, max(nb)), -1, dtype=np.int32)
    pool = np.full((NB, 2, B, Hkv, D), np.nan, dtype=np.float32)
    contig, k = [], 0
    for r in range(R):
        bt[r, :nb[r]] = perm[k:k + nb[r]]
        k += nb[r]
        Kc = rng.standard_normal((lens[r], Hkv, D)).astype(np.float32)
        Vc = rng.standard_normal((lens[r], Hkv, D)).astype(np.float32)
        contig.append((Kc, Vc))
        for j in range(lens[r]):  # place key j in block bt[r, j // B] at offset j % B
            pool[bt[r, j // B], 0, j % B] = Kc[j]
            pool[bt[r, j // B], 1, j % B] = Vc[j]
    if prefill:  # every request computes a trailing chunk of random size
        qlen = np.array([rng.integers(1, L, endpoint=True) for L in lens], dtype=np.int32)
    else:
        qlen = np.ones(R, dtype=np.int32)
    nc = (lens - qlen).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    problem = dict(q=q, pool=pool, block_table=bt, seq_lens=lens.astype(np.int32),
                   query_start_loc=qsl, num_computed=nc, scale=1.0 / math.sqrt(D),
                   dtype="f32")
    return contig, problem


def check_against_sdpa(seed=0, trials=6):
    """Textbook reduction: the paged oracle equals torch's scaled-dot-product
    attention (fp64, CPU) on the same keys laid out contiguously, with the
    causal offset mask and KV heads repeated per query group."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    for trial in range(trials):
        Hkv = [1, 2, 2, 4, 1, 3][trial % 6]
        G = [4, 2, 1, 2, 1, 2][trial % 6]
        contig, P = random_paged_problem(rng, Hq=Hkv * G, Hkv=Hkv, prefill=trial % 2 == 1)
        out = oracle.paged_attention(**P)
        qsl, nc = P["query_start_loc"], P["num_computed"]
        for r, (Kc, Vc) in enumerate(contig):
            t0, t1 = qsl[r], qsl[r + 1]
            L = Kc.shape[0]
            qt = torch.from_numpy(P["q"][t0:t1].astype(np.float64)).transpose(0, 1)[None]
            kt = torch.from_numpy(Kc.astype(np.float64)).transpose(0, 1)
            vt = torch.from_numpy(Vc.astype(np.float64)).transpose(0, 1)
            kt = kt.repeat_interleave(G, dim=0)[None]
            vt = vt.repeat_interleave(G, dim=0)[None]
            pos = nc[r] + np.arange(t1 - t0)
            mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
            want = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                  scale=P["scale"])
            want = want[0].transpose(0, 1).numpy()
            err = np.max(np.abs(out[t0:t1] - want))
            assert err < 1e-12, (trial, r, err)


def brute_force_attention(q, pool, bt, seq_lens, qsl, nc, scale, Hkv):
    """Element-by-element loops, written independently of the vectorised
    oracle: explicit block/offset walk, running max, exp, weighted sum."""
    T, Hq, D = q.shape
    B = pool.shape[2]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for r in range(len(seq_lens)):
        for t in range(int(qsl[r]), int(qsl[r + 1])):
            pos = int(nc[r]) + (t - int(qsl[r]))
            for h in range(Hq):
                g = h // G
                scores = []
                for j in range(pos + 1):
                    blk = int(bt[r][j // B])
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[t, h, d]) * float(pool[blk, 0, j % B, g, d])
                    scores.append(acc * scale)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for d in range(D):
                    acc = 0.0
                    for j in range(pos + 1):
                        blk = int(bt[r][j // B])
                        acc += w[j] * float(pool[blk, 1, j % B, g, d])
                    out[t, h, d] = acc / tot
    return out


def check_against_brute_force(seed=1, trials=4):
    rng = np.random.default_rng(seed)
    for trial in range(trials):
        _, P = random_paged_problem(rng, R=2, Hq=4, Hkv=2, D=4, B=4, NB=30, max_len=24,
                                    prefill=trial % 2 == 0)
        out = oracle.paged_attention(**P)
        want = brute_force_attention(P["q"], P["pool"], P["block_table"], P["seq_lens"],
                                     P["query_start_loc"], P["num_computed"], P["scale"],
                                     P["pool"].shape[3])
        err = np.max(np.abs(out - want))
        assert err < 1e-12, (trial, err)


def check_permutation_invariance(seed=2):
    """Relabelling physical blocks (moving pool blocks, mapping tables and
    slots) changes neither the attention result nor the scattered content."""
    rng = np.random.default_rng(seed)
    _, P = random_paged_problem(rng, R=4, NB=48, max_len=30, prefill=True)
    NB, B = P["pool"].shape[0], P["pool"].shape[2]
    perm = rng.permutation(NB)
    pool2 = np.empty_like(P["pool"])
    pool2[perm] = P["pool"]
    bt2 = np.where(P["block_table"] >= 0, perm[np.maximum(P["block_table"], 0)], -1)
    a = oracle.paged_attention(**P)
    b = oracle.paged_attention(**dict(P, pool=pool2, block_table=bt2.astype(np.int32)))
    assert np.array_equal(a, b)
    # scatter: slots follow the relabelling
    slots = oracle.slot_mapping(P["block_table"], P["query_start_loc"], P["num_computed"], B)
    slots2 = perm[slots // B] * B + slots % B
    T, Hkv, D = P["q"].shape[0], P["pool"].shape[3], P["pool"].shape[4]
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    s1 = oracle.reshape_and_cache(P["pool"], k, v, slots)
    s2 = oracle.reshape_and_cache(pool2, k, v, slots2)
    moved = np.empty_like(s1)
    moved[perm] = s1
    assert np.array_equal(moved, s2, equal_nan=True)


def check_special_cases(seed=3):
    rng = np.random.default_rng(seed)
    Hkv, G, D, B = 2, 2, 16, 4
    # (1) one key: the output is V_0 exactly
    _, P = random_paged_problem(rng, R=1, Hq=Hkv * G, Hkv=Hkv, D=D, B=B, max_len=1)
    out = oracle.paged_attention(**P)
    v0 = P["pool"][P["block_table"][0, 0], 1, 0].astype(np.float64)
    for h in range(Hkv * G):
        assert np.array_equal(out[0, h], v0[h // G])
    # (2) q = 0: uniform weights, the output is the mean of V_0..V_pos
    contig, P = random_paged_problem(rng, R=2, Hq=Hkv * G, Hkv=Hkv, D=D, B=B, max_len=30)
    P["q"][:] = 0
    out = oracle.paged_attention(**P)
    for r, (Kc, Vc) in enumerate(contig):
        mean = Vc.astype(np.float64).mean(axis=0)
        for h in range(Hkv * G):
            assert np.max(np.abs(out[r, h] - mean[h // G])) < 1e-13
    # (3) a dominant key: q = 100 K_k / |K_k| picks V_k
    contig, P = random_paged_problem(rng, R=1, Hq=Hkv * G, Hkv=Hkv, D=D, B=B, max_len=30)
    Kc, Vc = contig[0]
    L = Kc.shape[0]
    kk = int(rng.integers(0, L))
    for h in range(Hkv * G):
        kvec = Kc[kk, h // G].astype(np.float64)
        P["q"][0, h] = (100.0 * math.sqrt(D) * kvec / np.linalg.norm(kvec)).astype(np.float32)
    out = oracle.paged_attention(**P)
    for h in range(Hkv * G):
        assert np.max(np.abs(out[0, h] - Vc[kk, h // G])) < 1e-6
    # (4) decode output = last row of a full causal prefill of the same tokens
    contig, P = random_paged_problem(rng, R=1, Hq=Hkv * G, Hkv=Hkv, D=D, B=B, max_len=30)
    L = int(P["seq_lens"][0])
    qfull = rng.standard_normal((L, Hkv * G, D)).astype(np.float32)
    full = oracle.paged_attention(**dict(P, q=qfull, num_computed=np.array([0], np.int32),
                                         query_start_loc=np.array([0, L], np.int32)))
    dec = oracle.paged_attention(**dict(P, q=qfull[-1:], num_computed=np.array([L - 1], np.int32),
                                        query_start_loc=np.array([0, 1], np.int32)))
    assert np.max(np.abs(full[-1] - dec[0])) < 1e-13
    # ... and the first row of the prefill sees key 0 only: it is V_0
    for h in range(Hkv * G):
        assert np.array_equal(full[0, h], contig[0][1][0, h // G].astype(np.float64))


def check_chunked_prefill_equivalence(seed=4):
    """[P4] §4.2: a prompt prefilled in budget-sized chunks (254/254/254/238
    of 1000 tokens) gives the same rows as one full prefill."""
    rng = np.random.default_rng(seed)
    L, Hkv, G, D, B = 1000, 1, 2, 8, 16
    nb = -(-L // B)
    NB = nb + 7
    bt = rng.permutation(NB)[:nb].astype(np.int32)[None]
    pool = np.full((NB, 2, B, Hkv, D), np.nan, dtype=np.float32)
    pool[bt[0]] = rng.standard_normal((nb, 2, B, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((L, Hkv * G, D)).astype(np.float32)
    common = dict(pool=pool, block_table=bt, scale=0.3, dtype="f32")
    full = oracle.paged_attention(q=q, seq_lens=np.array([L], np.int32),
                                  query_start_loc=np.array([0, L], np.int32),
                                  num_computed=np.array([0], np.int32), **common)
    done = 0
    for n in oracle.chunk_schedule(L, 254):
        part = oracle.paged_attention(q=q[done:done + n], seq_lens=np.array([done + n], np.int32),
                                      query_start_loc=np.array([0, n], np.int32),
                                      num_computed=np.array([done], np.int32), **common)
        assert np.max(np.abs(part - full[done:done + n])) < 1e-12
        done += n
    assert done == L


def check_prefix_sharing_invariance(seed=5):
    """Requests whose tables share physical prefix blocks give the same result
    as with private copies of those blocks."""
    rng = np.random.default_rng(seed)
    R, S, B, Hkv, D = 3, 2, 4, 2, 8
    lens = np.array([11, 14, 9], np.int32)
    nb = [-(-int(L) // B) for L in lens]
    NB = S + sum(n - S for n in nb) + R * S + 4
    pool = rng.standard_normal((NB, 2, B, Hkv, D)).astype(np.float32)
    bt = np.full((R, max(nb)), -1, np.int32)
    nxt = S
    for r in range(R):
        bt[r, :S] = np.arange(S)
        bt[r, S:nb[r]] = np.arange(nxt, nxt + nb[r] - S)
        nxt += nb[r] - S
    bt_priv = bt.copy()
    for r in range(R):
        for j in range(S):
            pool[nxt] = pool[j]
            bt_priv[r, j] = nxt
            nxt += 1
    q = rng.standard_normal((R, 2 * Hkv, D)).astype(np.float32)
    args = dict(q=q, pool=pool, seq_lens=lens, query_start_loc=np.arange(R + 1, dtype=np.int32),
                num_computed=lens - 1, scale=0.35, dtype="f32")
    a = oracle.paged_attention(block_table=bt, **args)
    b = oracle.paged_attention(block_table=bt_priv, **args)
    assert np.array_equal(a, b)


def check_split_merge(seed=6):
    """Merging per-partition (max, sum, unnormalised output) triples gives the
    direct softmax result for any partition size."""
    rng = np.random.default_rng(seed)
    L, D = 1000, 16
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    qv = rng.standard_normal(D) * 3
    s = (K @ qv) * 0.25
    p = np.exp(s - s.max())
    direct = p @ V / p.sum()
    for part in (1, 7, 16, 333, 512, 1000, 4096):
        m, l, o = oracle.paged_attention_partials(qv, K, V, 0.25, part)
        assert m.size == -(-L // part)
        assert np.max(np.abs(oracle.merge_partials(m, l, o) - direct)) < 1e-12


def check_reshape_and_cache(seed=7):
    """[P4] §3.4 example: writing slot 193 stores the token at kv_cache[12, :, 1];
    every other byte of the pool is unchanged and slot -1 writes nothing."""
    rng = np.random.default_rng(seed)
    NB, B, H, D = 24, 16, 2, 8
    pool = rng.standard_normal((NB, 2, B, H, D)).astype(np.float32)
    k = rng.standard_normal((3, H, D)).astype(np.float32)
    v = rng.standard_normal((3, H, D)).astype(np.float32)
    out = oracle.reshape_and_cache(pool, k, v, np.array([193, -1, 144], np.int64))
    assert np.array_equal(out[12, 0, 1], k[0]) and np.array_equal(out[12, 1, 1], v[0])
    assert np.array_equal(out[9, 0, 0], k[2]) and np.array_equal(out[9, 1, 0], v[2])
    changed = np.argwhere(np.any(out != pool, axis=(3, 4)))
    assert sorted(map(tuple, changed.tolist())) == [(9, 0, 0), (9, 1, 0), (12, 0, 1), (12, 1, 1)]
    assert not np.array_equal(out, pool)
    # the input pool itself is untouched (the oracle returns a copy)
    fresh = np.random.default_rng(seed).standard_normal((NB, 2, B, H, D)).astype(np.float32)
    assert np.array_equal(pool, fresh)


def check_copy_on_write_fork(seed=9):
    """[P1] §4.3.2 (parallel sampling): three samples share prompt blocks
    [0, 1, 2]; before a sample writes into the shared, partly filled last
    block it gets a private copy (block 10, 20 or 30).  Pinned by the
    textbook result: each sample's attention after its own write equals plain
    softmax attention over the prompt's keys plus that sample's key, laid out
    contiguously; the shared blocks keep their bits."""
    rng = np.random.default_rng(seed)
    B, Hkv, G, D, NB = 16, 2, 2, 8, 40
    prompt = 2 * B + 14                       # last prompt block 14/16 full
    f32 = lambda shape: rng.standard_normal(shape).astype(np.float32)  # noqa: E731
    pool = f32((NB, 2, B, Hkv, D))
    K_p, V_p = f32((prompt, Hkv, D)), f32((prompt, Hkv, D))
    for j in range(prompt):                   # prompt blocks 0, 1, 2 in order
        pool[j // B, 0, j % B], pool[j // B, 1, j % B] = K_p[j], V_p[j]
    shared_before = pool[:3].copy()
    private = [10, 20, 30]
    forked = ref.copy_blocks(pool, np.array([[2, d] for d in private]))
    assert np.array_equal(forked[:3], shared_before)
    for d in private:
        assert np.array_equal(forked[d], pool[2])
    # every sample writes its own new token at position `prompt`
    k_new, v_new = f32((3, Hkv, D)), f32((3, Hkv, D))
    tables = np.array([[0, 1, d] for d in private], np.int32)
    qsl = np.arange(4, dtype=np.int32)
    slots = oracle.slot_mapping(tables, qsl, np.full(3, prompt, np.int32), B)
    assert list(slots) == [d * B + prompt - 2 * B for d in private]
    after = oracle.reshape_and_cache(forked, k_new, v_new, slots)
    assert np.array_equal(after[:3], shared_before)
    q = f32((3, Hkv * G, D))
    scale = 0.3
    got = oracle.paged_attention(q, after, tables, np.full(3, prompt + 1, np.int32), qsl,
                                 np.full(3, prompt, np.int32), scale, "f32")
    for smp in range(3):
        K = np.concatenate([K_p, k_new[smp:smp + 1]])
        V = np.concatenate([V_p, v_new[smp:smp + 1]])
        for h in range(Hkv * G):
            s = scale * (K[:, h // G].astype(np.float64) @ q[smp, h].astype(np.float64))
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ V[:, h // G].astype(np.float64)
            assert np.max(np.abs(got[smp, h] - want)) < 1e-12
    # the order of the copies does not matter, and rows with -1 are skipped
    rev = ref.copy_blocks(pool, np.array([[2, 30], [-1, 5], [2, 20], [2, 10]]))
    assert np.array_equal(rev, forked)
    for bad in ([[2, 10], [3, 10]], [[2, 10], [10, 11]]):
        try:
            ref.copy_blocks(pool, np.array(bad))
        except ValueError:
            continue
        raise AssertionError(f"precondition not enforced for {bad}")


def check_element_decoding():
    """bfloat16 is the upper 16 bits of an IEEE-754 binary32; binary16 per IEEE-754."""
    bf = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x3E80: 0.25, 0x0000: 0.0,
          0x7F7F: 3.3895313892515355e38, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133}
    got = oracle.decode_bits(np.array(list(bf), dtype=np.uint16), "bf16")
    assert np.array_equal(got, np.array(list(bf.values())))
    assert np.isinf(oracle.decode_bits(np.array([0x7F80], np.uint16), "bf16")[0])
    assert np.isnan(oracle.decode_bits(np.array([0x7FC0], np.uint16), "bf16")[0])
    hf = {0x3C00: 1.0, 0x7BFF: 65504.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x3555: 0.333251953125}
    got = oracle.decode_bits(np.array(list(hf), dtype=np.uint16), "f16")
    assert np.array_equal(got, np.array(list(hf.values())))


def check_bf16_paths_agree(seed=8):
    """The same problem stored as bf16 bits gives the f32 result on the
    bf16-representable values (decoding is used for q, K and V alike)."""
    rng = np.random.default_rng(seed)
    _, P = random_paged_problem(rng, R=3, prefill=True)
    def to_bf16_grid(x):
        u = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        return u.view(np.float32)
    Pf = dict(P, q=to_bf16_grid(P["q"]), pool=to_bf16_grid(P["pool"]))
    Pb = dict(P, q=(Pf["q"].view(np.uint32) >> 16).astype(np.uint16),
              pool=(Pf["pool"].view(np.uint32) >> 16).astype(np.uint16), dtype="bf16")
    a = oracle.paged_attention(**Pf)
    b = oracle.paged_attention(**Pb)
    assert np.array_equal(a, b, equal_nan=True)


def check_used_slot_mask():
    """The slots attention may read, against closed forms of the tables:
    with private blocks, logical block j of a request with L keys holds
    exactly its first min(16, L - 16 j) offsets and no other slot is used, so
    the count is sum(L); with a shared prefix of P blocks the prefix blocks
    are full and counted once, 16 P + sum(L - 16 P) in all."""
    from workloads import make_workload
    for name in ("tiny_f32_decode", "decode_bf16_small", "mixed_bf16_small",
                 "prefix_shared_small"):
        w = make_workload(name, values=False)
        B = w.block_size
        m = oracle.used_slot_mask(w.block_table, w.seq_lens, w.num_blocks, B)
        assert m.shape == (w.num_blocks, B)
        P = int(w.meta.get("shared_prefix_blocks", 0))
        owned = set()
        for r, L in enumerate(int(x) for x in w.seq_lens):
            for j in range(-(-L // B)):
                blk = int(w.block_table[r, j])
                n = min(B, L - j * B)
                assert m[blk, :n].all() and not m[blk, n:].any(), (name, r, j)
                owned.add(blk)
        others = np.setdiff1d(np.arange(w.num_blocks), np.array(sorted(owned)))
        assert not m[others].any(), name
        want = int(w.seq_lens.sum()) if P == 0 else \
            B * P + int((w.seq_lens - B * P).sum())
        assert int(m.sum()) == want, (name, int(m.sum()), want)


def check_validate_metadata():
    """The host-side metadata check accepts every committed workload and
    rejects each planted violation of a precondition the kernels trust
    ("vllm v1 源码精读（三）" §3.4 tables and slots, §4.2 packed offsets and
    computed counts)."""
    import meta_mutations as mm
    from workloads import make_workload
    for name in ("tiny_f32_decode", "decode_bf16_small", "mixed_bf16_small",
                 "prefix_shared_small", "long_decode_small", "mixed_chunked_prefill_bf16"):
        w = make_workload(name, values=False)
        oracle.validate_metadata(w.block_table, w.seq_lens, w.query_start_loc, w.num_computed,
                                 w.num_blocks, w.block_size, mm.slots_of(w))
    for label, w, slots, _flag in mm.mutations():
        try:
            oracle.validate_metadata(w.block_table, w.seq_lens, w.query_start_loc,
                                     w.num_computed, w.num_blocks, w.block_size, slots)
        except ValueError:
            continue
        raise AssertionError(f"validate_metadata accepted: {label}")
    # skipped tokens (negative slots) are not violations
    w = mm.mixed()
    s = mm.slots_of(w)
    s[::3] = -1
    oracle.validate_metadata(w.block_table, w.seq_lens, w.query_start_loc, w.num_computed,
                             w.num_blocks, w.block_size, s)


ALL_CHECKS = [
    check_slot_worked_example,
    check_pool_example_shapes,
    check_size_closed_forms,
    check_against_sdpa,
    check_against_brute_force,
    check_permutation_invariance,
    check_special_cases,
    check_chunked_prefill_equivalence,
    check_prefix_sharing_invariance,
    check_split_merge,
    check_reshape_and_cache,
    check_copy_on_write_fork,
    check_element_decoding,
    check_bf16_paths_agree,
    check_used_slot_mask,
    check_validate_metadata,
]
