"""Parity of the HIP path (through the C ABI) with the CPU oracle, on an MI355X.

Write: bit-exact over the whole cache.  Decode: within max-abs 1e-5 (fp32) or
2e-2 + 1e-2 |ref| (bf16) of the unrounded fp64 oracle, element by element.
Every case compares every output: the five full-size workloads compare the
write over the whole cache and the decode of every sequence, in the same
launch configuration the benchmark times (automatic partition size).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import CONFIG_ORDER, CONFIGS, SENTINEL, make_custom, make_workload
from tests.gpu_util import assert_matches_oracle, oracle_per_sequence, stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU-only machine)")
    pk.load_library()          # fails loudly if the HIP library is not built
    yield


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def _bits(a):
    """Bit patterns of stored values (NaN-safe equality)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _same_bits(t, ref):
    return np.array_equal(_bits(stored_np(t)), _bits(ref))


def _oracle_write(w):
    kc, vc = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(kc, vc, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    return kc, vc


def _run_write_decode(w, partition_size=0):
    """GPU write (in place on clones) then GPU decode; returns caches and out."""
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)
    out = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                    partition_size=partition_size)
    torch.cuda.synchronize()
    return kc, vc, out


# ---------------------------------------------------------------------------
# write
# ---------------------------------------------------------------------------

def test_write_padding_example_shape():
    """The page's write example (slots [4, 5, -1, 1], padding row of sentinels)
    on a geometry the kernels support (bs 8, D 64): bit-exact vs the oracle,
    no sentinel anywhere, the last slot untouched."""
    _say("write padding example")
    dev = torch.device("cuda")
    kc = torch.zeros(3, 8, 1, 64, device=dev)
    vc = torch.zeros_like(kc)
    k = torch.tensor([10.0, 20.0, 30.0, 40.0], device=dev).view(4, 1, 1).repeat(1, 1, 64)
    v = k * 0.1
    slots = torch.tensor([4, 5, -1, 1], dtype=torch.int64, device=dev)
    k[2] = SENTINEL
    v[2] = SENTINEL
    ko, vo = stored_np(kc).copy(), stored_np(vc).copy()
    O.write_kv(ko, vo, stored_np(k), stored_np(v), stored_np(slots))
    assert pk.write_kv(kc, vc, k, v, slots) is None
    torch.cuda.synchronize()
    assert np.array_equal(stored_np(kc).view(np.uint32), ko.view(np.uint32))
    assert np.array_equal(stored_np(vc).view(np.uint32), vo.view(np.uint32))
    assert int((kc == SENTINEL).sum()) == 0 and int((vc == SENTINEL).sum()) == 0
    assert float(kc[0, 4, 0, 0]) == 10.0 and float(kc[0, 1, 0, 0]) == 40.0
    assert int((kc[-1, -1] != 0).sum()) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D,KVH", [(64, 1), (128, 3), (256, 2)])
def test_write_random_geometry(dtype, D, KVH):
    """Random caches (not zeros), interleaved padding, shuffled slots: the whole
    cache after the write equals the oracle's bit for bit."""
    _say(f"write random {dtype} D={D} KVH={KVH}")
    w = make_custom(num_seqs=5, num_heads=KVH * 2, num_kv_heads=KVH, head_dim=D, block_size=8,
                    dtype=dtype, lens=[1, 8, 9, 30, 17], pad_tokens=3, seed=D + KVH, device="cuda")
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)
    torch.cuda.synchronize()
    ko, vo = _oracle_write(w)
    assert _same_bits(kc, ko) and _same_bits(vc, vo)


def test_write_zero_tokens_is_noop():
    w = make_custom(num_seqs=1, num_heads=2, num_kv_heads=1, head_dim=64, block_size=8,
                    lens=[3], seed=1, device="cuda")
    kc = w.k_cache.clone()
    pk.write_kv(kc, w.v_cache.clone(), w.k_new[:0], w.v_new[:0], w.slot_mapping[:0])
    torch.cuda.synchronize()
    assert torch.equal(kc, w.k_cache)


# ---------------------------------------------------------------------------
# decode, small cases (every output compared)
# ---------------------------------------------------------------------------

def test_tiny_f32_config_all_partitions():
    """The tiny fp32 workload (n = 1 and a multiple of 16 included, 99999 tails),
    write then decode, at the automatic and at forced small partition sizes."""
    w = make_workload(CONFIGS["tiny_f32"], "cuda")
    ko, vo = _oracle_write(w)
    ref = O.decode(stored_np(w.q), ko, vo, stored_np(w.block_tables), stored_np(w.context_lens),
                   w.scale, "f32")
    for P in (0, 16, 32, 64, 128):
        _say(f"tiny_f32 P={P}")
        kc, vc, out = _run_write_decode(w, P)
        assert _same_bits(kc, ko) and _same_bits(vc, vo)
        assert_matches_oracle(out, ref, "f32", f"tiny_f32 P={P}")


_SHAPES = [
    # dtype, D, bs, KVH, G
    ("f32", 64, 16, 2, 4),
    ("f32", 64, 8, 1, 8),
    ("f32", 128, 32, 2, 2),
    ("f32", 256, 8, 1, 3),
    ("bf16", 64, 8, 2, 4),
    ("bf16", 64, 16, 1, 1),
    ("bf16", 64, 64, 2, 8),
    ("bf16", 128, 16, 8, 4),
    ("bf16", 128, 8, 2, 6),
    ("bf16", 128, 32, 8, 8),
    ("bf16", 128, 64, 1, 16),
    ("bf16", 256, 16, 4, 4),
    ("bf16", 256, 32, 2, 5),
]


@pytest.mark.parametrize("dtype,D,bs,KVH,G", _SHAPES, ids=lambda x: str(x))
def test_random_shapes_poisoned(dtype, D, bs, KVH, G):
    """Random lengths (1, multiples of bs, others), shuffled blocks, every row no
    sequence reads filled with NaN, table tails pointing at NaN blocks; several
    partition sizes so that both the one-partition and the merge paths run."""
    lens = [1, bs, 3 * bs, 5 * bs + 3, 2 * bs - 1, 37, 300]
    w = make_custom(num_seqs=len(lens), num_heads=KVH * G, num_kv_heads=KVH, head_dim=D,
                    block_size=bs, dtype=dtype, lens=lens, tail="poison", poison=True,
                    pad_tokens=2, seed=D * 7 + bs + G, device="cuda")
    ko, vo = _oracle_write(w)
    ref = O.decode(stored_np(w.q), ko, vo, stored_np(w.block_tables), stored_np(w.context_lens),
                   w.scale, dtype)
    assert np.all(np.isfinite(ref))
    for P in sorted({0, bs, 2 * bs, 4 * bs, 64 if 64 % bs == 0 else bs}):
        _say(f"random {dtype} D={D} bs={bs} KVH={KVH} G={G} P={P}")
        kc, vc, out = _run_write_decode(w, P)
        assert _same_bits(kc, ko) and _same_bits(vc, vo)
        assert_matches_oracle(out, ref, dtype, f"{dtype} D{D} bs{bs} KVH{KVH} G{G} P{P}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_returns_v_row_exactly(dtype):
    """A one-token context returns that token's V row bit-exactly, whatever q is
    (the page's worked example, sequence 1)."""
    _say(f"n=1 exact {dtype}")
    w = make_custom(num_seqs=3, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                    dtype=dtype, lens=[1, 1, 1], seed=3, device="cuda")
    kc, vc, out = _run_write_decode(w)
    tbl = w.block_tables.long().cpu()
    for b in range(3):
        for h in range(8):
            row = vc[int(tbl[b, 0]), 0, h // 4]
            assert torch.equal(out[b, h].view(torch.int16 if dtype == "bf16" else torch.int32),
                               row.view(torch.int16 if dtype == "bf16" else torch.int32))


def test_zero_length_gives_zeros():
    """Reading for n = 0 (the pages imply n >= 1): the output is zeros."""
    _say("n=0")
    w = make_custom(num_seqs=3, num_heads=4, num_kv_heads=2, head_dim=64, block_size=8,
                    dtype="bf16", lens=[5, 1, 20], seed=4, device="cuda")
    lens = w.context_lens.clone()
    lens[1] = 0
    out = torch.full_like(w.q, 7.0)
    for P in (0, 8):
        pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, lens, w.scale, out=out, partition_size=P)
        torch.cuda.synchronize()
        assert int((out[1] != 0).sum()) == 0
        ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache),
                       stored_np(w.block_tables), stored_np(lens), w.scale, "bf16")
        assert_matches_oracle(out, ref, "bf16", f"n=0 P={P}")


def test_split_entry_points_equal_decode():
    """pa_decode_partials followed by pa_decode_merge gives pa_decode's result
    (both match the oracle; they run the same kernels, so bits agree)."""
    _say("split entry points")
    w = make_custom(num_seqs=4, num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                    dtype="bf16", lens=[700, 5, 129, 1000], seed=6, device="cuda")
    P = 64
    a = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, partition_size=P)
    ws = pk.new_workspace(4, 16, w.block_tables.shape[1], w.k_cache, P)
    b = torch.empty_like(w.q)
    pk.decode_partials(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, out=b,
                       workspace=ws, partition_size=P)
    pk.decode_merge(w.q, w.k_cache, w.block_tables, w.context_lens, out=b, workspace=ws,
                    partition_size=P)
    torch.cuda.synchronize()
    ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache),
                   stored_np(w.block_tables), stored_np(w.context_lens), w.scale, "bf16")
    assert_matches_oracle(a, ref, "bf16", "decode")
    assert_matches_oracle(b, ref, "bf16", "two-pass")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_reused_across_calls_and_sizes():
    """One workspace, with stale contents from earlier calls, serves repeated
    calls and other geometries: results are identical call after call."""
    _say("workspace reuse")
    big = torch.full((8 << 20,), 0x7F, dtype=torch.uint8, device="cuda")   # stale garbage
    for trial, (B, H, KVH, lens, P) in enumerate([
            (4, 16, 4, [700, 5, 129, 1000], 32),
            (6, 32, 8, [1, 300, 17, 64, 999, 250], 16),
            (2, 8, 2, [4000, 33], 64)]):
        w = make_custom(num_seqs=B, num_heads=H, num_kv_heads=KVH, head_dim=128, block_size=16,
                        dtype="bf16", lens=lens, seed=20 + trial, device="cuda")
        assert pk.workspace_bytes(B, H, w.block_tables.shape[1], w.k_cache, P) <= big.numel()
        ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache),
                       stored_np(w.block_tables), stored_np(w.context_lens), w.scale, "bf16")
        outs = []
        for rep in range(3):
            o = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale,
                          workspace=big, partition_size=P)
            torch.cuda.synchronize()
            assert_matches_oracle(o, ref, "bf16", f"reuse trial {trial} rep {rep}")
            outs.append(o.view(torch.int16).clone())
        assert all(torch.equal(outs[0], x) for x in outs[1:])


@pytest.mark.parametrize("B", [1000, 4100])
def test_many_sequences(B):
    """Many sequences of mixed lengths, every 7th with n = 0: up to 4096
    sequences the partial kernel runs as resident workgroups walking the list
    of existing (sequence, partition) pairs, found by a two-level search over
    the sequences; beyond that as one workgroup per unit."""
    _say(f"many sequences B={B}")
    lens = np.random.default_rng(B).integers(1, 200, size=B).tolist()
    w = make_custom(num_seqs=B, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                    dtype="bf16", lens=lens, seed=B % 97, device="cuda")
    ctx = w.context_lens.clone()
    ctx[::7] = 0
    ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache),
                   stored_np(w.block_tables), stored_np(ctx), w.scale, "bf16")
    for P in (0, 32, 64):
        out = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, ctx, w.scale, partition_size=P)
        torch.cuda.synchronize()
        assert_matches_oracle(out, ref, "bf16", f"B={B} P={P}")


def test_out_of_order_and_aliased_tables():
    """An out-of-order table (as in [3, 1]) and two tables aliasing the same
    physical blocks give the dense result for each sequence."""
    _say("aliased tables")
    w = make_custom(num_seqs=2, num_heads=4, num_kv_heads=1, head_dim=64, block_size=8,
                    dtype="f32", lens=[16, 16], seed=8, device="cuda")
    t = w.block_tables.clone()
    t[1, :2] = torch.flip(t[0, :2], [0])      # seq 1 reads seq 0's blocks in reverse order
    out = pk.decode(w.q, w.k_cache, w.v_cache, t, w.context_lens, w.scale)
    torch.cuda.synchronize()
    ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache), stored_np(t),
                   stored_np(w.context_lens), w.scale, "f32")
    assert_matches_oracle(out, ref, "f32", "aliased")


# ---------------------------------------------------------------------------
# full-size workloads: whole-cache write, every sequence's decode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", CONFIG_ORDER[1:])
def test_full_size_config(name):
    cfg = CONFIGS[name]
    _say(f"full {name}: generate")
    w = make_workload(cfg, "cuda")
    _say(f"full {name}: write + decode on GPU")
    kc, vc, out = _run_write_decode(w)
    _say(f"full {name}: oracle write")
    ko, vo = _oracle_write(w)
    assert _same_bits(kc, ko), "k_cache differs from the oracle's write"
    assert _same_bits(vc, vo), "v_cache differs from the oracle's write"
    q, tbl, lens = stored_np(w.q), stored_np(w.block_tables), stored_np(w.context_lens)
    _say(f"full {name}: oracle decode of all {len(lens)} sequences ({int(lens.sum())} tokens)")
    ref = oracle_per_sequence(lambda b0, b1: O.decode(q[b0:b1], ko, vo, tbl[b0:b1], lens[b0:b1], w.scale,
                                                      cfg.dtype), len(lens))
    err = assert_matches_oracle(out, ref, cfg.dtype, name)
    _say(f"full {name}: every output within tolerance, max err {err:.2e}")


def test_graph_replay_of_write_and_decode():
    """The write and both decode kernels captured in one HIP graph and
    replayed: every replay, with eager work on the stream between replays,
    gives the eager result (the library enqueues kernels only)."""
    _say("graph replay")
    w = make_custom(num_seqs=6, num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                    dtype="bf16", lens=[1, 40, 300, 1100, 2500, 17], seed=77, device="cuda")
    B, H, W = w.q.shape[0], w.q.shape[1], w.block_tables.shape[1]
    P = 256
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    # the new rows are written at each sequence's last position
    k_new = torch.randn(B, 4, 128, device="cuda").to(torch.bfloat16)
    v_new = torch.randn(B, 4, 128, device="cuda").to(torch.bfloat16)
    lens = w.context_lens.cpu().tolist()
    tbl = w.block_tables.cpu()
    slots = torch.tensor([int(tbl[b, (n - 1) // 16]) * 16 + (n - 1) % 16 for b, n in enumerate(lens)],
                         dtype=torch.int64, device="cuda")
    ws = pk.new_workspace(B, H, W, kc, P)
    out = torch.empty_like(w.q)

    def step():
        pk.write_kv(kc, vc, k_new, v_new, slots)
        pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, out=out, workspace=ws,
                  partition_size=P)

    ko, vo = stored_np(kc).copy(), stored_np(vc).copy()
    O.write_kv(ko, vo, stored_np(k_new), stored_np(v_new), stored_np(slots))
    ref = O.decode(stored_np(w.q), ko, vo, stored_np(w.block_tables), stored_np(w.context_lens),
                   w.scale, "bf16")
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    eager = out.clone()
    assert_matches_oracle(eager, ref, "bf16", "eager step")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.empty(1 << 24, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        junk.normal_()                              # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert np.array_equal(stored_np(kc), ko) and np.array_equal(stored_np(vc), vo)


@pytest.mark.parametrize("cfg_name", ["tiny_f32", "llama3_8b_bf16"])
def test_graph_step_padded_batch_new_inputs_each_replay(cfg_name):
    """A decode step as a serving loop runs it: write + decode captured once
    in a HIP graph over fixed buffers (a padded batch: slot -1 rows carry the
    sentinel and must not be written), then replayed with new q, k, v and
    slots copied into those buffers before each replay.  Every replay is held
    to the oracle: the write bit for bit over the whole cache, the decode
    within the tolerance."""
    cfg = CONFIGS[cfg_name]
    w = make_workload(cfg, "cuda")
    _say(f"graph step {cfg_name}")
    B, H, D = w.q.shape
    W = w.block_tables.shape[1]
    T = w.slot_mapping.numel()
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    ws = pk.new_workspace(B, H, W, kc)
    q_buf, k_buf, v_buf = w.q.clone(), w.k_new.clone(), w.v_new.clone()
    slot_buf = w.slot_mapping.clone()
    out = torch.empty_like(w.q)

    def step():
        pk.write_kv(kc, vc, k_buf, v_buf, slot_buf)
        pk.decode(q_buf, kc, vc, w.block_tables, w.context_lens, w.scale, out=out, workspace=ws)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()                                       # warm the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gen = torch.Generator(device="cuda").manual_seed(321)
    pad = slot_buf < 0
    for rep in range(3):
        # new inputs in place: fresh q, k, v rows; the valid slots permuted among themselves
        q_buf.copy_(torch.randn(q_buf.shape, generator=gen, device="cuda").to(q_buf.dtype))
        k_buf.copy_(torch.randn(k_buf.shape, generator=gen, device="cuda").to(k_buf.dtype))
        v_buf.copy_(torch.randn(v_buf.shape, generator=gen, device="cuda").to(v_buf.dtype))
        k_buf[pad] = SENTINEL
        v_buf[pad] = SENTINEL
        valid = torch.nonzero(~pad).flatten()
        perm = valid[torch.randperm(valid.numel(), generator=gen, device="cuda")]
        new_slots = slot_buf.clone()
        new_slots[valid] = slot_buf[perm]
        slot_buf.copy_(new_slots)
        ko, vo = stored_np(kc).copy(), stored_np(vc).copy()
        O.write_kv(ko, vo, stored_np(k_buf), stored_np(v_buf), stored_np(slot_buf))
        ref = O.decode(stored_np(q_buf), ko, vo, stored_np(w.block_tables), stored_np(w.context_lens),
                       w.scale, cfg.dtype)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(kc, ko) and _same_bits(vc, vo), f"{cfg_name} replay {rep}: write"
        err = assert_matches_oracle(out, ref, cfg.dtype, f"{cfg_name} replay {rep}")
        _say(f"graph step {cfg_name} replay {rep} (T={T}, {int(pad.sum())} padding rows): max err {err:.2e}")


def test_graph_replay_of_prefill_and_shared_prefix_decode():
    """pa_prefill (planning kernel, which zeroes its own ticket counters, then
    the persistent attention kernel) and pa_decode_shared_prefix (the table
    check, shared units and the merge) captured in one HIP graph: every
    replay, with eager work between replays, gives the eager result bit for
    bit, and that result matches the oracle."""
    _say("graph replay: prefill + shared-prefix decode")
    from synth import make_prefill_custom
    wp = make_prefill_custom(num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, cached=[0, 100, 37],
                             new=[70, 33, 129], dtype="bf16", seed=78, device="cuda")
    kc, vc = wp.k_cache.clone(), wp.v_cache.clone()
    pk.write_kv(kc, vc, wp.k_new, wp.v_new, wp.slot_mapping)
    T, H, _ = wp.q.shape
    pws = pk.prefill_workspace(3, H, wp.block_tables.shape[1], T, kc)
    pout = torch.empty_like(wp.q)
    lens = [300, 129, 200, 140, 1000, 128, 70, 0, 400]
    wd = make_custom(num_seqs=9, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                     lens=lens, seed=79, device="cuda")
    tbl = wd.block_tables.cpu().clone()
    tbl[:, :8] = tbl[0, :8]                                   # a common 128-token prefix
    wd.block_tables = tbl.cuda()
    B, W = 9, wd.block_tables.shape[1]
    dws = pk.new_workspace(B, H, W, wd.k_cache, 64)
    dout = torch.empty_like(wd.q)

    def step():
        pk.prefill(wp.q, kc, vc, wp.block_tables, wp.context_lens, wp.query_start_loc, wp.scale, out=pout,
                   workspace=pws)
        pk.decode_shared_prefix(wd.q, wd.k_cache, wd.v_cache, wd.block_tables, wd.context_lens, wd.scale, 128,
                                out=dout, workspace=dws, partition_size=64)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    pe, de = pout.clone(), dout.clone()
    ko, vo = stored_np(kc), stored_np(vc)
    assert_matches_oracle(pe, O.prefill(stored_np(wp.q), ko, vo, stored_np(wp.block_tables),
                                        stored_np(wp.context_lens), stored_np(wp.query_start_loc), wp.scale,
                                        "bf16"), "bf16", "eager prefill")
    assert_matches_oracle(de, O.decode(stored_np(wd.q), stored_np(wd.k_cache), stored_np(wd.v_cache),
                                       stored_np(wd.block_tables), stored_np(wd.context_lens), wd.scale, "bf16"),
                          "bf16", "eager shared-prefix decode")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.empty(1 << 24, device="cuda")
    for rep in range(4):
        pout.fill_(float("nan"))
        dout.fill_(float("nan"))
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pout.view(torch.int16), pe.view(torch.int16)), f"prefill replay {rep}"
        assert torch.equal(dout.view(torch.int16), de.view(torch.int16)), f"decode replay {rep}"


@pytest.mark.parametrize("B", [15, 16, 17, 33, 48, 63, 64, 65, 127, 129])
def test_unit_list_across_lane_rows_and_chunks(B):
    """The persistent kernel's unit list takes prefix sums of each sequence's
    full partitions over 64-lane chunks of the batch, 16 lanes to a row.
    Batch sizes on both sides of the row and chunk edges, with one-block
    partitions so that the counts run into the hundreds (and some sequences
    have none: n <= P, or n = 0), must give the oracle's result for every
    sequence, with the partials + merge halves bit-equal to the one call."""
    rng = np.random.default_rng(1000 + B)
    lens = [int(x) for x in rng.integers(1, 700, B)]
    lens[B // 2] = 0
    lens[-1] = 16
    w = make_custom(num_seqs=B, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                    lens=lens, seed=B, device="cuda")
    ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache), stored_np(w.block_tables),
                   stored_np(w.context_lens), w.scale, "bf16")
    W = w.block_tables.shape[1]
    for P in (16, 48):
        out = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, partition_size=P)
        ws = pk.new_workspace(B, 8, W, w.k_cache, P)
        two = torch.empty_like(w.q)
        pk.decode_partials(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, out=two,
                           workspace=ws, partition_size=P)
        pk.decode_merge(w.q, w.k_cache, w.block_tables, w.context_lens, out=two, workspace=ws, partition_size=P)
        torch.cuda.synchronize()
        err = assert_matches_oracle(out, ref, "bf16", f"B={B} P={P}")
        assert torch.equal(two.view(torch.int16), out.view(torch.int16)), f"B={B} P={P}: two calls differ"
        _say(f"unit list B={B} P={P}: max err {err:.2e}")
