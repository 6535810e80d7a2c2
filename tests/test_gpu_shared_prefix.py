"""pa_decode_shared_prefix on an MI355X, held to the oracle: batches whose
tables begin with row 0's blocks (a common prompt, as on "PagedAttention
kernel：paged KV cache 与 block table", 面试官追问) decoded with the shared
partitions folded several sequences at a time.

Each case mixes sequences that take part (same leading entries, longer than
the shared partitions) with ones that must not: a context that ends inside or
exactly at the shared part, an empty context, and a table that differs from
row 0 in one shared entry.  The hint is also given wrong (too long, zero) and
for shapes that cannot use it (G = 3, G = 16, fp32), where the call must
still equal the oracle.  All outputs are compared with the fp64 oracle within
the dtype's tolerance; the partials + merge halves must equal the one-call
form bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import CONFIGS, make_custom, make_workload, to_vllm_layout
from tests.gpu_util import assert_matches_oracle, oracle_per_sequence, stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[gpu-shared-prefix] {msg}", flush=True)
    sys.stdout.flush()


def _share(w, rows, k, differ=()):
    """Point the first k entries of each table row in `rows` at row 0's blocks
    (and, for rows in `differ`, change entry k // 2 back to its own block)."""
    tbl = w.block_tables.cpu().clone()
    for b in rows:
        own = tbl[b, k // 2].item()
        tbl[b, :k] = tbl[0, :k]
        if b in differ:
            tbl[b, k // 2] = own if own != tbl[0, k // 2].item() else (own + 1) % w.num_blocks
    w.block_tables = tbl.to(w.block_tables.device)
    return w


def _oracle(w, kc=None, vc=None):
    kc = stored_np(w.k_cache) if kc is None else kc
    vc = stored_np(w.v_cache) if vc is None else vc
    return O.decode(stored_np(w.q), kc, vc, stored_np(w.block_tables), stored_np(w.context_lens), w.scale,
                    w.cfg.dtype)


def _run(w, shared, P, k_cache=None, v_cache=None):
    kc = w.k_cache if k_cache is None else k_cache
    vc = w.v_cache if v_cache is None else v_cache
    B, H, _ = w.q.shape
    W = w.block_tables.shape[1]
    ws = pk.new_workspace(B, H, W, kc, P)
    out = pk.decode_shared_prefix(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, shared,
                                  workspace=ws, partition_size=P)
    torch.cuda.synchronize()
    return out, ws


# (H, KVH, D, bs, P, shared tokens, lengths, rows sharing, rows differing in one entry)
CASES = [
    # G = 4: groups of 4 sequences; 2 shared partitions of 64; sequence 5 ends at the
    # shared part (128), 6 inside it, 7 is empty, 8 differs in one shared entry
    (8, 2, 128, 16, 64, 128, [300, 129, 200, 140, 1000, 128, 70, 0, 400, 260, 131],
     range(11), (8,)),
    # G = 8: pairs of sequences; 3 partitions of 32 shared (hint 100 -> 96 tokens), bs 8
    (16, 2, 64, 8, 32, 100, [97, 500, 96, 150, 99, 33, 256], range(7), ()),
    # G = 2: 8 sequences per unit; D 256, bs 32
    (4, 2, 256, 32, 64, 128, [129, 190, 1024, 300, 64, 700, 129, 140, 150, 200], range(10), (3,)),
    # G = 1: 16 sequences per unit, 20 sequences -> groups of 16 and 4
    (4, 4, 128, 16, 128, 256, [257 + 13 * i for i in range(20)], range(20), ()),
    # only some rows share; the rest are ordinary
    (8, 2, 128, 16, 64, 192, [500, 400, 300, 250, 600, 193], (0, 2, 4, 5), ()),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[0]}_KVH{c[1]}_D{c[2]}_bs{c[3]}_P{c[4]}_S{c[5]}")
def test_shared_prefix_matches_oracle(case):
    H, KVH, D, bs, P, shared, lens, rows, differ = case
    w = make_custom(num_seqs=len(lens), num_heads=H, num_kv_heads=KVH, head_dim=D, block_size=bs,
                    dtype="bf16", lens=lens, seed=H * D + bs, device="cuda")
    w = _share(w, rows, -(-shared // bs), differ)
    ref = _oracle(w)
    out, _ = _run(w, shared, P)
    err = assert_matches_oracle(out, ref, "bf16", f"shared prefix H{H} D{D} bs{bs}")
    # the same call without the hint, and the two-call form
    plain = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, partition_size=P)
    assert_matches_oracle(plain, ref, "bf16", "pa_decode")
    B, H_, _ = w.q.shape
    ws = pk.new_workspace(B, H_, w.block_tables.shape[1], w.k_cache, P)
    two = torch.empty_like(w.q)
    pk.decode_partials_shared_prefix(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, shared,
                                     out=two, workspace=ws, partition_size=P)
    pk.decode_merge(w.q, w.k_cache, w.block_tables, w.context_lens, out=two, workspace=ws, partition_size=P)
    torch.cuda.synchronize()
    assert torch.equal(two.view(torch.int16), out.view(torch.int16)), "partials + merge differ from one call"
    _say(f"H{H} KVH{KVH} D{D} bs{bs} P{P} shared {shared}: max err {err:.2e}")


def test_many_sequences_and_a_hint_covering_the_table():
    """200 sequences (several 64-sequence passes of the list, 50 groups of 4),
    a few of them too short or with one differing entry; then a hint as long
    as the whole table: 6 partitions of 64 (384 tokens) are shared, which only
    row 0 (399 tokens, its own entries) passes, as a group of one."""
    rng = np.random.default_rng(9)
    lens = [int(x) for x in rng.integers(1, 400, 200)]
    lens[0] = 399
    w = _share(make_custom(num_seqs=200, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype="bf16",
                           lens=lens, seed=31, device="cuda"), range(200), 8, (7, 100, 199))
    ref = _oracle(w)
    out, _ = _run(w, 128, 64)
    assert_matches_oracle(out, ref, "bf16", "200 sequences")
    W = w.block_tables.shape[1]
    out, _ = _run(w, W * 16, 64)
    assert_matches_oracle(out, ref, "bf16", "hint = whole table")


@pytest.mark.parametrize("hint", [0, 16, 4096, 1 << 30])
def test_wrong_or_useless_hints(hint):
    """A hint of nothing, less than a partition, or beyond every table: the
    result is still the oracle's."""
    lens = [300, 129, 200, 140, 1000, 128]
    w = _share(make_custom(num_seqs=6, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                           lens=lens, seed=17, device="cuda"), range(6), 8)
    out, _ = _run(w, hint, 64)
    assert_matches_oracle(out, _oracle(w), "bf16", f"hint {hint}")


@pytest.mark.parametrize("H,KVH,dtype", [(6, 2, "bf16"), (32, 2, "bf16"), (8, 2, "f32")])
def test_shapes_that_cannot_share(H, KVH, dtype):
    """G = 3 (does not divide 16), G = 16 (no room for a second sequence) and
    fp32 caches fall back to the ordinary decode."""
    lens = [300, 200, 129, 400]
    w = _share(make_custom(num_seqs=4, num_heads=H, num_kv_heads=KVH, head_dim=64, block_size=16, dtype=dtype,
                           lens=lens, seed=H, device="cuda"), range(4), 8)
    out, _ = _run(w, 128, 64)
    assert_matches_oracle(out, _oracle(w), dtype, f"H{H} KVH{KVH} {dtype}")


def test_vllm_layout():
    lens = [300, 129, 200, 140, 1000, 128, 70, 0, 400]
    w = _share(make_custom(num_seqs=9, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                           lens=lens, seed=23, device="cuda"), range(9), 8, (2,))
    kp, vp = to_vllm_layout(w.k_cache, w.v_cache)
    out, _ = _run(w, 128, 64, kp, vp)
    assert_matches_oracle(out, _oracle(w), "bf16", "vLLM layout")


def test_prefix_shared_workload_full_size():
    """The 128-sequence prefix-shared workload (2048 shared tokens, D 256) at
    the automatic partition size, as the benchmark runs it: every sequence
    against the oracle, and against pa_decode."""
    w = make_workload(CONFIGS["prefix_shared_bf16"], "cuda")
    B, H, D = w.q.shape
    W = w.block_tables.shape[1]
    P = pk.partition_size(B, H, W, w.k_cache)
    out, _ = _run(w, 2048, P)
    plain = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    torch.cuda.synchronize()
    kc, vc = stored_np(w.k_cache), stored_np(w.v_cache)
    q, tbl, lens = stored_np(w.q), stored_np(w.block_tables), stored_np(w.context_lens)
    ref = oracle_per_sequence(lambda b0, b1: O.decode(q[b0:b1], kc, vc, tbl[b0:b1], lens[b0:b1], w.scale, "bf16"),
                              B)
    err = assert_matches_oracle(out, ref, "bf16", "prefix_shared_bf16 (shared units)")
    err_plain = assert_matches_oracle(plain, ref, "bf16", "prefix_shared_bf16 (pa_decode)")
    diff = (out.float() - plain.float()).abs()
    _say(f"prefix_shared_bf16: P {P}, all {B} sequences: max err {err:.2e} (pa_decode {err_plain:.2e}), "
         f"max |shared - plain| {float(diff.max()):.2e}")


@pytest.mark.parametrize("extra", [0, 1, 2, 3, "misaligned"])
def test_table_check_widths_and_alignment(extra):
    """The shared-prefix table check reads 4 entries per load when the rows
    are 16-byte aligned and one otherwise: table widths W of every residue
    mod 4 (tails filled with 99999), and a table whose first entry is not
    16-byte aligned, give the oracle's result; a row differing in the last
    shared entry is caught by both forms."""
    lens = [300, 129, 200, 140, 1000, 128, 70, 0, 400, 260, 131]
    w = make_custom(num_seqs=len(lens), num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                    lens=lens, seed=91, device="cuda")
    w = _share(w, range(len(lens)), 8, ())
    tbl = w.block_tables.cpu().clone()
    tbl[3, 7] = (tbl[3, 7] + 1) % w.num_blocks          # the last shared entry differs for row 3
    B, W = tbl.shape
    pad = 0 if extra == "misaligned" else (4 - W % 4 + extra) % 4
    wide = torch.full((B, W + pad), 99999, dtype=torch.int32)
    wide[:, :W] = tbl
    if extra == "misaligned":
        store = torch.zeros(B * W + 1, dtype=torch.int32, device="cuda")
        t = store[1:].view(B, W)
        t.copy_(wide.cuda())
        assert t.is_contiguous() and t.data_ptr() % 16 != 0
        w.block_tables = t
    else:
        w.block_tables = wide.cuda()
    ref = _oracle(w)
    out, _ = _run(w, 128, 64)
    err = assert_matches_oracle(out, ref, "bf16", f"table width {w.block_tables.shape[1]} ({extra})")
    _say(f"table width {w.block_tables.shape[1]} ({extra}): max err {err:.2e}")


@pytest.mark.parametrize("case", ["two_passes", "row_wider_than_workgroup"])
def test_table_check_passes_and_wide_rows(case):
    """The table check's two quad forms. With rows of 384 shared entries (96
    quads) a 512-thread workgroup keeps one quad column per thread over 5 rows
    at a time (32 threads idle), 80 rows per pass: 96 sequences take a second
    pass, whose rows 85 and 95 differ from row 0 in the first and last shared
    entry.  With rows of 2112 shared entries (528 quads, more than the
    workgroup has threads) the check falls back to the (sequence, quad) walk.
    Both give the oracle's result."""
    rng = np.random.default_rng(23)
    if case == "two_passes":
        bs, P, shared = 16, 1024, 6144
        lens = [int(x) for x in rng.integers(6145, 6657, 96)]
        lens[0], lens[5], lens[6], lens[7] = 6656, 6144, 100, 0
        differ = {3: 192, 85: 0, 95: 383}
    else:
        bs, P, shared = 8, 512, 16896
        lens = [17120, 17000, 16950, 16897, 16896, 5000]
        differ = {2: 2111, 3: 1000}
    w = make_custom(num_seqs=len(lens), num_heads=8, num_kv_heads=2, head_dim=64, block_size=bs, dtype="bf16",
                    lens=lens, seed=57, device="cuda")
    spb = shared // P * P // bs
    w = _share(w, range(len(lens)), spb, ())
    tbl = w.block_tables.cpu().clone()
    for b, j in differ.items():
        tbl[b, j] = (tbl[b, j] + 1) % w.num_blocks
    w.block_tables = tbl.to(w.block_tables.device)
    B, W = tbl.shape
    assert W % 4 == 0 and w.block_tables.data_ptr() % 16 == 0, "the quad forms need 16-byte aligned rows"
    quads = -(-spb // 4)
    assert (quads <= 512) == (case == "two_passes")
    ref = _oracle(w)
    out, _ = _run(w, shared, P)
    err = assert_matches_oracle(out, ref, "bf16", f"table check {case}")
    _say(f"table check {case}: {B} sequences, {spb} shared entries ({quads} quads), max err {err:.2e}")
