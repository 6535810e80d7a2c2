"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an oracle module ``O`` (the real one, or a deliberately
broken copy made by ``tests/test_oracle_mutants.py``) and raises if ``O``
disagrees with the pages' printed values, a closed form, an invariant or a
brute-force computation done here by other means.

Pages cited:
  [P1] "P09 · Paged KV 写入 + decode attention（参考实现）" (kuanzhou.online)
  [P2] "PagedAttention kernel：paged KV cache 与 block table"
       (inference-learning-path.pages.dev)
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# helpers local to the pins (independent of the oracle's own code)
# ---------------------------------------------------------------------------

def _dense_attention_loops(q, K, V, scale):
    """Dense single-query attention, scalar Python loops and math.exp (brute
    force for tiny inputs).  q [D], K [n, D], V [n, D] as nested floats."""
    n, D = len(K), len(q)
    s = [scale * sum(q[d] * K[j][d] for d in range(D)) for j in range(n)]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    tot = sum(w)
    return [sum(w[j] * V[j][d] for j in range(n)) / tot for d in range(D)]


def _paged_from_dense(rng, Ks, Vs, bs, extra_blocks, tail_value):
    """Place per-sequence contiguous K/V ([n, KVH, D] each) into a randomly
    permuted block pool, token by token.  Unused positions hold NaN.
    Returns k_cache, v_cache, block_tables (tails = tail_value), context_lens."""
    KVH, D = Ks[0].shape[1], Ks[0].shape[2]
    nbs = [-(-k.shape[0] // bs) for k in Ks]
    NB = sum(nbs) + extra_blocks
    perm = rng.permutation(NB)
    W = max(max(nbs), 1) + 2
    kc = np.full((NB, bs, KVH, D), np.nan)
    vc = np.full((NB, bs, KVH, D), np.nan)
    tables = np.full((len(Ks), W), tail_value, dtype=np.int64)
    nxt = 0
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        for j in range(nbs[b]):
            phys = int(perm[nxt])
            nxt += 1
            tables[b, j] = phys
            for t in range(bs):
                tok = j * bs + t
                if tok < K.shape[0]:
                    kc[phys, t] = K[tok]
                    vc[phys, t] = V[tok]
    lens = np.array([k.shape[0] for k in Ks], dtype=np.int64)
    return kc.astype(np.float32), vc.astype(np.float32), tables, lens


def _f32(x):
    return np.asarray(x, dtype=np.float32)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_bf16_widening(O):
    """Every bf16 bit pattern widens to the value torch assigns it (an
    independent implementation), NaNs to NaN."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # A few by hand: 1.0, -2.0, 0.25, pi rounded, smallest subnormal 2^-133, inf.
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x3E80: 0.25, 0x4049: 3.140625,
            0x0001: 2.0 ** -133, 0x7F80: math.inf}
    for b, val in hand.items():
        assert O.bf16_bits_to_f64(np.array([b], dtype=np.uint16))[0] == val


def pin_m1_write_example(O):
    """[P1] L1 hints, 例 1: the printed cache after a write with padding."""
    g = _load("m1_write_example.json")
    kc = np.zeros(g["cache_shape"], dtype=np.float32)
    vc = np.zeros(g["cache_shape"], dtype=np.float32)
    k = _f32(g["k"]).reshape(-1, 1, 1)
    v = (k * np.float32(g["v_factor"])).astype(np.float32)
    ret = O.write_kv(kc, vc, k, v, np.array(g["slot_mapping"], dtype=np.int64))
    assert ret is None
    assert np.array_equal(kc[:, :, 0, 0], _f32(g["k_cache_expected"]))
    assert np.array_equal(vc[:, :, 0, 0], _f32(g["v_cache_expected"]))
    assert not np.any(kc == g["absent_value"])          # invariant I1
    assert not np.any(vc == np.float32(g["absent_value"]) * np.float32(g["v_factor"]))


def _m2_inputs(O):
    g = _load("m2_decode_example.json")
    NB, bs, KVH, D = g["num_blocks"], g["block_size"], g["num_kv_heads"], g["head_dim"]
    kc = np.zeros((NB, bs, KVH, D), dtype=np.float32)
    vc = np.zeros((NB, bs, KVH, D), dtype=np.float32)
    k = _f32(g["seq0_k"] + g["seq1_k"]).reshape(-1, KVH, D)
    v = _f32(g["seq0_v"] + g["seq1_v"]).reshape(-1, KVH, D)
    O.write_kv(kc, vc, k, v, np.array(g["seq0_slots"] + g["seq1_slots"], dtype=np.int64))
    q = _f32([g["q_seq0"], g["q_seq1"]])
    tables = np.array(g["block_tables"], dtype=np.int64)
    lens = np.array(g["context_lens"], dtype=np.int64)
    return g, q, kc, vc, tables, lens


def pin_m2_decode_example(O):
    """[P1] 逐步图 例 2: printed result to the page's 4 decimals, plus the
    closed forms behind it (weights (a, b, a) with 2a + b = 1 give exactly
    [3, 4]; head 1 gives ((1 + 8e^2), (2 + 10e^2)) / (1 + 2e^2); a one-token
    sequence returns its V row exactly)."""
    g, q, kc, vc, tables, lens = _m2_inputs(O)
    # the write itself, as the figure draws the blocks
    assert np.array_equal(kc[2, :, 0], _f32([[1, 0], [0, 1]]))
    assert np.array_equal(kc[0, 0, 0], _f32([1, 1]))
    assert np.array_equal(kc[3, 0, 0], _f32([2, 2]))
    out = O.decode(q, kc, vc, tables, lens, g["scale"], "f32")
    assert out.dtype == np.float64 and out.shape == (2, 2, 2)
    tol = 0.5 * 10.0 ** -g["printed_digits"]
    assert np.allclose(out, np.array(g["printed_result"]), atol=tol, rtol=0)
    assert np.allclose(out[0, 0], [3.0, 4.0], atol=1e-12, rtol=0)
    e2 = math.exp(2.0)
    exact = [(1 + 8 * e2) / (1 + 2 * e2), (2 + 10 * e2) / (1 + 2 * e2)]
    assert np.allclose(out[0, 1], exact, atol=1e-12, rtol=0)
    assert np.array_equal(out[1], np.array([[7.0, 8.0], [7.0, 8.0]]))
    # The printed probabilities follow from the printed scores.
    for key, scores in g["printed_scores"].items():
        s = np.array(scores)
        p = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
        assert np.allclose(p, g["printed_probs"][key], atol=tol, rtol=0)


def pin_m2_gather_truncation(O):
    """[P1] 例 2 steps 3-4: the untruncated gather has a 4th row (block 0,
    offset 1); truncation keeps exactly n = 3 rows (invariant I3).  Without
    truncation the zero row would get weight e^0 and head 0 would read
    [(6e + 3)/(2e + 2), (8e + 4)/(2e + 2)] ~ [2.5966, 3.4621] instead."""
    g, q, kc, vc, tables, lens = _m2_inputs(O)
    rows = O.gather_context(kc, tables[0], 3)
    assert rows.shape == (3, 1, 2)
    assert np.array_equal(rows[:, 0, :], _f32(g["printed_gathered_seq0_untruncated"][:3]))
    out = O.decode(q, kc, vc, tables, lens, 1.0, "f32")
    e = math.e
    wrong = [(6 * e + 3) / (2 * e + 2), (8 * e + 4) / (2 * e + 2)]
    assert abs(out[0, 0, 0] - wrong[0]) > 0.3


def pin_gqa_map(O):
    """Invariant I5 and 例 3: H=4, KVH=2 -> [0,0,1,1]; H=8, KVH=2 ->
    [0,0,0,0,1,1,1,1]; and the decode itself uses that map (each kv head's
    single V row identifies it)."""
    assert [O.kv_head_of(h, 4, 2) for h in range(4)] == [0, 0, 1, 1]
    assert [O.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    for H, KVH in ((8, 2), (6, 3), (4, 4), (4, 1)):
        D, bs = 2, 4
        kc = np.zeros((2, bs, KVH, D), dtype=np.float32)
        vc = np.zeros((2, bs, KVH, D), dtype=np.float32)
        for c in range(KVH):
            vc[1, 0, c] = [c + 1.0, -(c + 1.0)]
        q = np.ones((1, H, D), dtype=np.float32)
        out = O.decode(q, kc, vc, np.array([[1, 7]]), np.array([1]), 1.0, "f32")
        G = H // KVH
        expect = [h // G for h in range(H)]
        assert [int(round(out[0, h, 0])) - 1 for h in range(H)] == expect


def pin_slot_arithmetic(O):
    """[P1] 关键问题 / L3 answers: slot 7 with bs 4 is block 1 offset 3;
    n = 5 with bs 4 uses 2 table entries = 8 positions, 3 cut off; the flat
    slot index equals block * bs + offset for every slot (细节)."""
    assert O.slot_to_block_offset(7, 4) == (1, 3)
    assert O.blocks_needed(5, 4) == 2 and O.blocks_needed(8, 4) == 2
    assert O.blocks_needed(1, 16) == 1 and O.blocks_needed(16, 16) == 1 and O.blocks_needed(17, 16) == 2
    for bs in (1, 2, 4, 16):
        for s in range(3 * bs):
            blk, off = O.slot_to_block_offset(s, bs)
            assert blk * bs + off == s and 0 <= off < bs
    # writing slot s lands on row s of the flattened cache
    NB, bs = 3, 4
    for s in range(NB * bs):
        kc = np.zeros((NB, bs, 1, 1), dtype=np.float32)
        vc = np.zeros_like(kc)
        O.write_kv(kc, vc, _f32([[[5.0]]]), _f32([[[6.0]]]), np.array([s]))
        assert np.flatnonzero(kc.reshape(-1)).tolist() == [s]
        assert np.flatnonzero(vc.reshape(-1)).tolist() == [s]
    # n = 5, bs = 4: exactly 5 rows come back, from the table's first 2 entries
    kc = np.arange(3 * 4 * 1 * 1, dtype=np.float32).reshape(3, 4, 1, 1)
    rows = O.gather_context(kc, np.array([2, 0, 99999]), 5)
    assert rows[:, 0, 0].tolist() == [8.0, 9.0, 10.0, 11.0, 0.0]


def pin_i1_padding_not_written(O):
    """Invariant I1: a padding token whose values are all the sentinel 9.0
    leaves no 9.0 anywhere, in particular not in the last slot (where a -1
    index would land)."""
    rng = np.random.default_rng(11)
    NB, bs, KVH, D = 5, 4, 2, 3
    kc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    vc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    k0, v0 = kc.copy(), vc.copy()
    T = 6
    k = rng.standard_normal((T, KVH, D)).astype(np.float32)
    v = rng.standard_normal((T, KVH, D)).astype(np.float32)
    slots = np.array([3, -1, 17, -1, 0, NB * bs - 2])
    k[slots < 0] = 9.0
    v[slots < 0] = 9.0
    O.write_kv(kc, vc, k, v, slots)
    assert (kc == 9).sum() == 0 and (vc == 9).sum() == 0
    assert np.array_equal(kc[-1, -1], k0[-1, -1]) and np.array_equal(vc[-1, -1], v0[-1, -1])
    # every other row is untouched, every written row holds its token bit-exactly
    flat_k, flat_k0 = kc.reshape(NB * bs, KVH, D), k0.reshape(NB * bs, KVH, D)
    written = {int(s): i for i, s in enumerate(slots) if s >= 0}
    for s in range(NB * bs):
        want = k[written[s]] if s in written else flat_k0[s]
        assert np.array_equal(flat_k[s].view(np.uint32), want.view(np.uint32))


def pin_i2_table_tail_not_read(O):
    """Invariant I2: table tails of 99999 (beyond the pool) are never read;
    tails pointing at NaN-filled blocks do not reach the output."""
    rng = np.random.default_rng(12)
    KVH, D, bs = 1, 3, 4
    Ks = [rng.standard_normal((n, KVH, D)) for n in (5, 8, 1)]
    Vs = [rng.standard_normal((n, KVH, D)) for n in (5, 8, 1)]
    kc, vc, tables, lens = _paged_from_dense(rng, Ks, Vs, bs, extra_blocks=2, tail_value=99999)
    q = rng.standard_normal((3, 2, D)).astype(np.float32)
    out = O.decode(q, kc, vc, tables, lens, 0.5, "f32")
    assert np.all(np.isfinite(out))
    spare = [b for b in range(kc.shape[0]) if b not in set(tables[tables < kc.shape[0]].tolist())]
    t2 = tables.copy()
    for b in range(3):
        nb = -(-int(lens[b]) // bs)
        t2[b, nb:] = spare[0]
    kc[spare[0]] = np.nan
    vc[spare[0]] = np.nan
    out2 = O.decode(q, kc, vc, t2, lens, 0.5, "f32")
    assert np.array_equal(out, out2)


def pin_i3_exactly_n_rows(O):
    """Invariant I3: for n not a multiple of bs, the rows past n in the last
    block (here NaN) take no part; the gather returns exactly n rows."""
    rng = np.random.default_rng(13)
    bs, KVH, D = 4, 2, 3
    for n in (1, 3, 4, 5, 7, 8, 9):
        Ks = [rng.standard_normal((n, KVH, D))]
        Vs = [rng.standard_normal((n, KVH, D))]
        kc, vc, tables, lens = _paged_from_dense(rng, Ks, Vs, bs, extra_blocks=1, tail_value=99999)
        assert O.gather_context(kc, tables[0], n).shape == (n, KVH, D)
        q = rng.standard_normal((1, 4, D)).astype(np.float32)
        out = O.decode(q, kc, vc, tables, lens, 1.0, "f32")
        assert np.all(np.isfinite(out)), n


def pin_i4_dense_brute_force(O):
    """Invariant I4 / 自检: paged decode equals dense attention over the
    contiguous K/V (computed here with scalar loops), for random lengths
    (1, multiples of bs, others), random block sizes, GQA groups, shuffled
    physical blocks and garbage tails; fp64 agreement to 1e-12."""
    rng = np.random.default_rng(14)
    for trial in range(12):
        bs = int(rng.choice([1, 2, 3, 4, 8]))
        KVH = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4]))
        H, D = KVH * G, int(rng.choice([1, 2, 5]))
        lens = [1, bs * int(rng.integers(1, 4)), int(rng.integers(1, 13))]
        Ks = [rng.standard_normal((n, KVH, D)).astype(np.float32).astype(np.float64) for n in lens]
        Vs = [rng.standard_normal((n, KVH, D)).astype(np.float32).astype(np.float64) for n in lens]
        kc, vc, tables, cl = _paged_from_dense(rng, Ks, Vs, bs, extra_blocks=3, tail_value=77777)
        q = rng.standard_normal((len(lens), H, D)).astype(np.float32)
        scale = float(rng.uniform(0.1, 1.5))
        out = O.decode(q, kc, vc, tables, cl, scale, "f32")
        for b, n in enumerate(lens):
            for h in range(H):
                c = h // G
                ref = _dense_attention_loops(
                    [float(x) for x in q[b, h]],
                    [[float(x) for x in Ks[b][j, c]] for j in range(n)],
                    [[float(x) for x in Vs[b][j, c]] for j in range(n)], scale)
                assert np.allclose(out[b, h], ref, atol=1e-12, rtol=1e-12), (trial, b, h)


def pin_bf16_decode_dense(O):
    """The bf16 path of the oracle widens the stored patterns exactly: a bf16
    cache equals the f32 decode of the same values (each bf16 value is an
    exact f32), which brute force checks above."""
    rng = np.random.default_rng(15)
    NB, bs, KVH, D, H = 6, 4, 2, 8, 4
    vals = torch.from_numpy(rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)).to(torch.bfloat16)
    vals2 = torch.from_numpy(rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)).to(torch.bfloat16)
    qv = torch.from_numpy(rng.standard_normal((2, H, D)).astype(np.float32)).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    f32 = lambda t: t.to(torch.float32).numpy()
    tables = np.array([[3, 1, 99999], [5, 0, 2]])
    lens = np.array([6, 9])
    a = O.decode(bits(qv), bits(vals), bits(vals2), tables, lens, 0.3, "bf16")
    b = O.decode(f32(qv), f32(vals), f32(vals2), tables, lens, 0.3, "f32")
    assert np.array_equal(a, b)


def pin_fold_matches_direct(O):
    """[P2] 代码: the block-table walk with an online-softmax fold gives the
    same result as the direct softmax (to fp64 rounding), including an
    out-of-order table such as [3, 1] and a one-token sequence."""
    rng = np.random.default_rng(16)
    NB, bs, KVH, D, H = 5, 4, 2, 3, 4
    kc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    vc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    q = rng.standard_normal((3, H, D)).astype(np.float32)
    tables = np.array([[3, 1, 99999], [0, 99999, 99999], [4, 2, 1]])
    lens = np.array([7, 1, 12])
    a = O.decode(q, kc, vc, tables, lens, 0.7, "f32")
    b = O.decode_online_fold(q, kc, vc, tables, lens, 0.7, "f32")
    assert np.allclose(a, b, atol=1e-12, rtol=1e-12)


def pin_scale_before_softmax(O):
    """[P1] L3 answers: the scale multiplies the scores before the softmax.
    Two tokens with raw scores (2, 0) and values (1, 0): the output is the
    first token's weight, 1 / (1 + e^(-2 scale)) — a scale applied after the
    softmax would instead give scale * 1 / (1 + e^(-2))."""
    kc = np.zeros((1, 2, 1, 1), dtype=np.float32)
    vc = np.zeros((1, 2, 1, 1), dtype=np.float32)
    kc[0, 0, 0, 0], kc[0, 1, 0, 0] = 2.0, 0.0
    vc[0, 0, 0, 0], vc[0, 1, 0, 0] = 1.0, 0.0
    q = np.ones((1, 1, 1), dtype=np.float32)
    for scale in (0.25, 1.0, 3.0):
        out = O.decode(q, kc, vc, np.array([[0]]), np.array([2]), scale, "f32")
        assert abs(out[0, 0, 0] - 1.0 / (1.0 + math.exp(-2.0 * scale))) < 1e-14


def pin_n_zero_and_errors(O):
    """Readings: n = 0 gives zeros; an in-use table entry outside the pool,
    or a slot beyond the pool, is an error (not silently wrapped)."""
    kc = np.ones((2, 2, 1, 2), dtype=np.float32)
    q = np.ones((2, 1, 2), dtype=np.float32)
    out = O.decode(q, kc, kc, np.array([[0], [1]]), np.array([0, 2]), 1.0, "f32")
    assert np.array_equal(out[0], np.zeros((1, 2))) and np.array_equal(out[1], np.ones((1, 2)))
    import pytest
    with pytest.raises(O.OracleError):
        O.decode(q, kc, kc, np.array([[0], [5]]), np.array([1, 1]), 1.0, "f32")
    with pytest.raises(O.OracleError):
        O.write_kv(kc.copy(), kc.copy(), np.ones((1, 1, 2), np.float32), np.ones((1, 1, 2), np.float32), np.array([4]))
    with pytest.raises(O.OracleError):
        O.write_kv(kc.copy(), kc.copy(), np.ones((2, 1, 2), np.float32), np.ones((2, 1, 2), np.float32), np.array([1, 1]))


# ---------------------------------------------------------------------------
# prefill pins (the varlen version [P1] 面试官追问 asks for; [P1] 细节: decode
# needs no causal mask because its single query is the newest token)
# ---------------------------------------------------------------------------

def _prefill_case(rng, lens, qlens, KVH, G, D, bs, tail_value=55555):
    """Random paged case: per-sequence contiguous K/V placed in a shuffled
    pool, packed queries [T, H, D] and query_start_loc."""
    Ks = [rng.standard_normal((n, KVH, D)).astype(np.float32).astype(np.float64) for n in lens]
    Vs = [rng.standard_normal((n, KVH, D)).astype(np.float32).astype(np.float64) for n in lens]
    kc, vc, tables, cl = _paged_from_dense(rng, Ks, Vs, bs, extra_blocks=2, tail_value=tail_value)
    T = int(sum(qlens))
    q = rng.standard_normal((T, KVH * G, D)).astype(np.float32)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int64)
    return Ks, Vs, kc, vc, tables, cl, q, qs


def pin_prefill_brute_force(O):
    """Causal attention of each new query over the tokens up to its own
    position, with the key/value rows found by walking the table token by
    token (block table[j // bs], offset j % bs) and scalar Python loops; fp64
    agreement to 1e-12.  Lengths cover 1, multiples of bs and others; query
    counts cover 0, 1, all of the context and a part of it."""
    rng = np.random.default_rng(31)
    for trial in range(8):
        bs = int(rng.choice([1, 2, 3, 4]))
        KVH = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3]))
        D = int(rng.choice([1, 3, 4]))
        lens = [1, bs * int(rng.integers(1, 4)), int(rng.integers(2, 11)), int(rng.integers(1, 9))]
        qlens = [1, lens[1], int(rng.integers(1, lens[2])), 0]
        Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, lens, qlens, KVH, G, D, bs)
        scale = float(rng.uniform(0.2, 1.3))
        out = O.prefill(q, kc, vc, tables, cl, qs, scale, "f32")
        H = KVH * G
        for b, n in enumerate(lens):
            for i in range(qlens[b]):
                p = n - qlens[b] + i
                row = int(qs[b]) + i
                for h in range(H):
                    c = h // G
                    keys, vals = [], []
                    for j in range(p + 1):
                        blk = int(tables[b][j // bs])
                        keys.append([float(x) for x in kc[blk, j % bs, c]])
                        vals.append([float(x) for x in vc[blk, j % bs, c]])
                    ref = _dense_attention_loops([float(x) for x in q[row, h]], keys, vals, scale)
                    assert np.allclose(out[row, h], ref, atol=1e-12, rtol=1e-12), (trial, b, i, h)


def pin_prefill_one_query_is_decode(O):
    """With one new query per sequence the query is the newest token and sees
    the whole context: prefill reduces to decode ([P1] 细节), which the
    decode pins fix.  Agreement to 1e-13."""
    rng = np.random.default_rng(32)
    lens = [1, 5, 8, 13]
    Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, lens, [1, 1, 1, 1], KVH=2, G=2, D=4, bs=4)
    a = O.prefill(q, kc, vc, tables, cl, qs, 0.7, "f32")
    b = O.decode(q, kc, vc, tables, cl, 0.7, "f32")
    assert np.allclose(a, b, atol=1e-13, rtol=1e-13)


def pin_prefill_zero_keys_running_mean(O):
    """Closed form: with every key zero all visible scores are equal, so the
    softmax is uniform and query at position p returns the mean of V rows
    0..p.  A mask that is off by one, aligned to the first token instead of
    the last, or missing changes the mean."""
    rng = np.random.default_rng(33)
    lens, qlens = [7, 9], [7, 4]
    Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, lens, qlens, KVH=1, G=2, D=3, bs=2)
    kc = np.zeros_like(kc)
    out = O.prefill(q, kc, vc, tables, cl, qs, 1.0, "f32")
    for b, n in enumerate(lens):
        for i in range(qlens[b]):
            p = n - qlens[b] + i
            want = Vs[b][: p + 1, 0].mean(axis=0)
            for h in range(2):
                assert np.allclose(out[qs[b] + i, h], want, atol=1e-14), (b, i, h)


def pin_prefill_first_token_is_v0(O):
    """A fresh prefill (all n tokens new): the first query sees only token 0,
    so its output is exactly V[0] (weight 1), whatever q and K hold."""
    rng = np.random.default_rng(34)
    Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, [6], [6], KVH=2, G=1, D=4, bs=4)
    q = (q * 50).astype(np.float32)
    out = O.prefill(q, kc, vc, tables, cl, qs, 1.0, "f32")
    for h in range(2):
        assert np.array_equal(out[0, h], Vs[0][0, h])


def pin_prefill_chunk_invariance(O):
    """Chunked prefill: the same tokens' queries computed in two calls (the
    first c tokens with context c, then the rest with context n) give what one
    call over all n gives; position, not chunking, decides what a query sees."""
    rng = np.random.default_rng(35)
    n, c = 11, 4
    Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, [n], [n], KVH=1, G=3, D=5, bs=3)
    whole = O.prefill(q, kc, vc, tables, cl, qs, 0.9, "f32")
    first = O.prefill(q[:c], kc, vc, tables, np.array([c]), np.array([0, c]), 0.9, "f32")
    rest = O.prefill(q[c:], kc, vc, tables, np.array([n]), np.array([0, n - c]), 0.9, "f32")
    assert np.allclose(np.concatenate([first, rest]), whole, atol=1e-13, rtol=1e-13)


def pin_prefill_sdpa_fp64(O):
    """Library routine: torch's scaled_dot_product_attention in float64 on the
    dense per-sequence K/V, with an explicit boolean mask (query row i may
    see keys 0 .. n - L + i) and the kv heads expanded by repeat_interleave."""
    import torch.nn.functional as F
    rng = np.random.default_rng(36)
    lens, qlens = [12, 5, 9], [5, 5, 1]
    KVH, G, D = 2, 4, 8
    Ks, Vs, kc, vc, tables, cl, q, qs = _prefill_case(rng, lens, qlens, KVH, G, D, bs=4)
    out = O.prefill(q, kc, vc, tables, cl, qs, 0.35, "f32")
    for b, n in enumerate(lens):
        L = qlens[b]
        qt = torch.from_numpy(q[qs[b]:qs[b + 1]].astype(np.float64)).transpose(0, 1)       # [H, L, D]
        kt = torch.from_numpy(Ks[b]).transpose(0, 1).repeat_interleave(G, dim=0)          # [H, n, D]
        vt = torch.from_numpy(Vs[b]).transpose(0, 1).repeat_interleave(G, dim=0)
        mask = torch.arange(n)[None, :] <= (n - L + torch.arange(L))[:, None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.35)
        assert np.allclose(out[qs[b]:qs[b + 1]], ref.transpose(0, 1).numpy(), atol=1e-12, rtol=1e-12), b


def pin_prefill_errors(O):
    """Preconditions: more new queries than context tokens, or a
    query_start_loc that does not run from 0 to T, are errors."""
    import pytest
    kc = np.ones((2, 2, 1, 2), dtype=np.float32)
    q = np.ones((3, 1, 2), dtype=np.float32)
    with pytest.raises(O.OracleError):
        O.prefill(q, kc, kc, np.array([[0]]), np.array([2]), np.array([0, 3]), 1.0, "f32")
    with pytest.raises(O.OracleError):
        O.prefill(q, kc, kc, np.array([[0, 1]]), np.array([4]), np.array([1, 3]), 1.0, "f32")


# ---------------------------------------------------------------------------
# vLLM cache layout pins ([P2] 深入原理)
# ---------------------------------------------------------------------------

def pin_vllm_layout_indexing(O):
    """Element (blk, t, h, d) of [P1]'s layout sits at K[blk, h, d // x, t, d % x]
    and V[blk, h, d, t] of vLLM's, with x = 8 for 2-byte elements and 4 for
    4-byte ones (16 bytes per group); checked element by element with scalar
    loops, and unpacking inverts packing."""
    assert O.vllm_pack_width("bf16") == 8 and O.vllm_pack_width("f32") == 4
    rng = np.random.default_rng(41)
    for dtype, D in (("f32", 8), ("bf16", 16)):
        NB, bs, KVH = 3, 4, 2
        c = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
        if dtype == "bf16":
            c = torch.from_numpy(c).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        x = 8 if dtype == "bf16" else 4
        kp, vp = O.pack_k_vllm(c, dtype), O.pack_v_vllm(c)
        assert kp.shape == (NB, KVH, D // x, bs, x) and vp.shape == (NB, KVH, D, bs)
        for blk in range(NB):
            for t in range(bs):
                for h in range(KVH):
                    for d in range(D):
                        assert kp[blk, h, d // x, t, d % x] == c[blk, t, h, d]
                        assert vp[blk, h, d, t] == c[blk, t, h, d]
        assert np.array_equal(O.unpack_k_vllm(kp), c) and np.array_equal(O.unpack_v_vllm(vp), c)
        # the K group of 8 (bf16) or 4 (fp32) elements is 16 contiguous bytes
        assert kp.strides[-1] * x == 16 and kp.strides[-2] == 16


def pin_vllm_layout_write_and_decode(O):
    """The same write and decode on caches in vLLM's layout: the written values
    land where the layout says (scalar loop over the written slots), and the
    decode equals [P1]'s decode of the same values (it is attention either way,
    [P2] 直接答案)."""
    rng = np.random.default_rng(42)
    NB, bs, KVH, D, H = 6, 4, 2, 8, 4
    kc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    vc = rng.standard_normal((NB, bs, KVH, D)).astype(np.float32)
    k = rng.standard_normal((3, KVH, D)).astype(np.float32)
    v = rng.standard_normal((3, KVH, D)).astype(np.float32)
    slots = np.array([5, -1, 22])
    kp, vp = O.pack_k_vllm(kc, "f32"), O.pack_v_vllm(vc)
    O.write_kv_vllm(kp, vp, k, v, slots)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, t = s // bs, s % bs
        for h in range(KVH):
            for d in range(D):
                assert kp[blk, h, d // 4, t, d % 4] == k[i, h, d] and vp[blk, h, d, t] == v[i, h, d]
    tables = np.array([[1, 5, 77], [0, 2, 3]])
    lens = np.array([7, 12])
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    a = O.decode_vllm(q, kp, vp, tables, lens, 0.4, "f32")
    kw, vw = kc.copy(), vc.copy()
    O.write_kv(kw, vw, k, v, slots)
    b = O.decode(q, kw, vw, tables, lens, 0.4, "f32")
    assert np.array_equal(a, b)


ALL_PINS = [
    pin_bf16_widening,
    pin_m1_write_example,
    pin_m2_decode_example,
    pin_m2_gather_truncation,
    pin_gqa_map,
    pin_slot_arithmetic,
    pin_i1_padding_not_written,
    pin_i2_table_tail_not_read,
    pin_i3_exactly_n_rows,
    pin_i4_dense_brute_force,
    pin_bf16_decode_dense,
    pin_fold_matches_direct,
    pin_scale_before_softmax,
    pin_n_zero_and_errors,
    pin_prefill_brute_force,
    pin_prefill_one_query_is_decode,
    pin_prefill_zero_keys_running_mean,
    pin_prefill_first_token_is_v0,
    pin_prefill_chunk_invariance,
    pin_prefill_sdpa_fp64,
    pin_prefill_errors,
    pin_vllm_layout_indexing,
    pin_vllm_layout_write_and_decode,
]
