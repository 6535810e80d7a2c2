"""Parity of the HIP write and decode on caches in vLLM's layout (K
[NB, KVH, D/x, bs, x], V [NB, KVH, D, bs]; "PagedAttention kernel：paged KV
cache 与 block table", 深入原理) with the CPU oracle.

The GPU caches are the same seeded values as the P09-layout tests, moved
into vLLM's layout; expected values come from the oracle's own packing
(`pack_k_vllm` / `pack_v_vllm`) and its layout-aware write and decode.  The
write is compared bit for bit over both whole caches, the decode within the
bf16 tolerance, element by element.
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
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU-only machine)")
    pk.load_library()
    yield


def _say(msg):
    print(f"[gpu-vllm] {msg}", flush=True)
    sys.stdout.flush()


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _oracle(w):
    """Oracle caches after the write, in vLLM's layout (packed by the oracle)."""
    kp = O.pack_k_vllm(stored_np(w.k_cache), w.cfg.dtype)
    vp = O.pack_v_vllm(stored_np(w.v_cache))
    O.write_kv_vllm(kp, vp, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    return kp, vp


def _gpu_write(w):
    kc, vc = to_vllm_layout(w.k_cache, w.v_cache)
    pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)
    torch.cuda.synchronize()
    return kc, vc


@pytest.mark.parametrize("name", ["tiny_f32", "llama3_8b_bf16", "big_batch_bf16"])
def test_write_vllm_layout_config(name):
    """The scatter into vLLM's layout, bit-exact over both whole caches
    (fp32 and bf16; the large-batch config has 64 padding slots)."""
    w = make_workload(CONFIGS[name], "cuda")
    kc, vc = _gpu_write(w)
    kp, vp = _oracle(w)
    assert np.array_equal(_bits(stored_np(kc)), _bits(kp)), "k_cache"
    assert np.array_equal(_bits(stored_np(vc)), _bits(vp)), "v_cache"


# (D, bs, KVH, G, lengths): block sizes 8 (a tile spans two blocks), 16, 32;
# lengths 1, block multiples, ragged tails, several partitions.
CASES = [
    (128, 16, 2, 4, [1, 16, 37, 300, 1000]),
    (128, 8, 2, 4, [1, 8, 9, 63, 200]),
    (128, 32, 4, 2, [5, 32, 100, 513]),
    (64, 16, 2, 8, [3, 64, 250]),
    (256, 16, 2, 4, [17, 48, 700]),
    (128, 16, 1, 16, [33, 129]),
    # blocks of 32 and 64 tokens: 32-token tiles (head_dim <= 128), tile edges straddled
    (64, 32, 2, 8, [1, 31, 32, 33, 95, 400]),
    (128, 64, 2, 4, [1, 63, 64, 65, 300, 1030]),
    (128, 32, 2, 16, [31, 64, 96, 777]),
    (256, 32, 2, 4, [7, 33, 500]),              # head_dim 256 keeps 16-token tiles
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"D{c[0]}_bs{c[1]}_KVH{c[2]}_G{c[3]}")
@pytest.mark.parametrize("partition_size", [0, 64])
def test_decode_vllm_layout_poisoned(case, partition_size):
    """Write then decode in vLLM's layout on shuffled, NaN-poisoned pools
    (every row no sequence reads is NaN) with 99999 table tails."""
    D, bs, KVH, G, lens = case
    if partition_size and partition_size % bs:
        pytest.skip("partition must be a block multiple")
    w = make_custom(num_seqs=len(lens), num_heads=KVH * G, num_kv_heads=KVH, head_dim=D, block_size=bs,
                    dtype="bf16", lens=lens, seed=D + bs + KVH, device="cuda", poison=True)
    kc, vc = _gpu_write(w)
    out = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, partition_size=partition_size)
    torch.cuda.synchronize()
    kp, vp = _oracle(w)
    assert np.array_equal(stored_np(kc), kp) and np.array_equal(stored_np(vc), vp), "write"
    ref = O.decode_vllm(stored_np(w.q), kp, vp, stored_np(w.block_tables), stored_np(w.context_lens),
                        w.scale, "bf16")
    err = assert_matches_oracle(out, ref, "bf16", f"vllm D{D} bs{bs} P{partition_size}")
    _say(f"D{D} bs{bs} KVH{KVH} G{G} P{partition_size}: max err {err:.2e}")


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "long_ctx_bf16", "prefix_shared_bf16"])
def test_decode_vllm_layout_full_size(name):
    """Full-size configs in vLLM's layout, in the launch the benchmark times:
    the write over both whole caches, the decode of every sequence (the
    oracle's decode_vllm, with the caches unpacked once for all sequences)."""
    cfg = CONFIGS[name]
    w = make_workload(cfg, "cuda")
    kc, vc = _gpu_write(w)
    out = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale)
    torch.cuda.synchronize()
    kp, vp = _oracle(w)
    assert np.array_equal(stored_np(kc), kp) and np.array_equal(stored_np(vc), vp), "write"
    ku, vu = O.unpack_k_vllm(kp), O.unpack_v_vllm(vp)
    q, tbl, lens = stored_np(w.q), stored_np(w.block_tables), stored_np(w.context_lens)
    ref = oracle_per_sequence(lambda b0, b1: O.decode(q[b0:b1], ku, vu, tbl[b0:b1], lens[b0:b1], w.scale, "bf16"),
                              len(lens))
    err = assert_matches_oracle(out, ref, "bf16", name)
    _say(f"{name}: all {len(lens)} sequences within tolerance, max err {err:.2e}")


def test_decode_vllm_matches_p09_layout_kernel():
    """The two layouts' kernels on the same values: both within the oracle's
    tolerance, and within bf16 rounding of each other."""
    w = make_workload(CONFIGS["llama3_8b_bf16"], "cuda")
    kc, vc = _gpu_write(w)
    a = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale)
    k1, v1 = w.k_cache.clone(), w.v_cache.clone()
    pk.write_kv(k1, v1, w.k_new, w.v_new, w.slot_mapping)
    b = pk.decode(w.q, k1, v1, w.block_tables, w.context_lens, w.scale)
    torch.cuda.synchronize()
    assert (a.float() - b.float()).abs().max().item() <= 2e-2


# fp32 caches in vLLM's layout (x = 4 elements per 16-byte K group): the
# vector-ALU decode kernel (D, bs, KVH, G, lengths)
F32_CASES = [
    (64, 16, 2, 4, [1, 16, 40, 200, 193]),
    (128, 8, 2, 3, [1, 8, 9, 77, 300]),
    (256, 32, 1, 2, [5, 32, 33, 500]),
    (64, 64, 4, 1, [63, 64, 65, 1000]),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: f"f32_D{c[0]}_bs{c[1]}_KVH{c[2]}_G{c[3]}")
@pytest.mark.parametrize("partition_size", [0, 64])
def test_decode_vllm_layout_f32(case, partition_size):
    """fp32 write then decode in vLLM's layout on NaN-poisoned pools with
    99999 table tails, held to the fp32 tolerance (max-abs 1e-5)."""
    D, bs, KVH, G, lens = case
    if partition_size and partition_size % bs:
        pytest.skip("partition must be a block multiple")
    w = make_custom(num_seqs=len(lens), num_heads=KVH * G, num_kv_heads=KVH, head_dim=D, block_size=bs,
                    dtype="f32", lens=lens, seed=D + bs + KVH + 1, device="cuda", poison=True)
    kc, vc = _gpu_write(w)
    out = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, partition_size=partition_size)
    torch.cuda.synchronize()
    kp, vp = _oracle(w)
    assert np.array_equal(_bits(stored_np(kc)), _bits(kp)) and np.array_equal(_bits(stored_np(vc)), _bits(vp))
    ref = O.decode_vllm(stored_np(w.q), kp, vp, stored_np(w.block_tables), stored_np(w.context_lens), w.scale,
                        "f32")
    err = assert_matches_oracle(out, ref, "f32", f"f32 vllm D{D} bs{bs} P{partition_size}")
    _say(f"f32 D{D} bs{bs} KVH{KVH} G{G} P{partition_size}: max err {err:.2e}")


def test_tiny_f32_config_vllm_layout():
    """The tiny fp32 workload (n = 1 and 192 included, one -1 padding row) in
    vLLM's layout: write bit for bit, decode at several partition sizes."""
    w = make_workload(CONFIGS["tiny_f32"], "cuda")
    kc, vc = _gpu_write(w)
    kp, vp = _oracle(w)
    assert np.array_equal(_bits(stored_np(kc)), _bits(kp)) and np.array_equal(_bits(stored_np(vc)), _bits(vp))
    ref = O.decode_vllm(stored_np(w.q), kp, vp, stored_np(w.block_tables), stored_np(w.context_lens), w.scale,
                        "f32")
    for P in (0, 16, 48, 128):
        out = pk.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, partition_size=P)
        torch.cuda.synchronize()
        assert_matches_oracle(out, ref, "f32", f"tiny_f32 vllm P={P}")


def test_prefill_and_append_vllm_layout_f32():
    """fp32 prefill (one decode per query row) and the fp32 append step on
    caches in vLLM's layout."""
    from synth import make_new_rows, make_prefill_custom
    wp = make_prefill_custom(num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, cached=[0, 37, 200],
                             new=[20, 33, 9], dtype="f32", seed=71, device="cuda", poison=True)
    kc, vc = to_vllm_layout(wp.k_cache, wp.v_cache)
    pk.write_kv(kc, vc, wp.k_new, wp.v_new, wp.slot_mapping)
    out = pk.prefill(wp.q, kc, vc, wp.block_tables, wp.context_lens, wp.query_start_loc, wp.scale)
    torch.cuda.synchronize()
    ko, vo = stored_np(wp.k_cache).copy(), stored_np(wp.v_cache).copy()
    O.write_kv(ko, vo, stored_np(wp.k_new), stored_np(wp.v_new), stored_np(wp.slot_mapping))
    assert np.array_equal(_bits(stored_np(kc)), _bits(O.pack_k_vllm(ko, "f32")))
    ref = O.prefill(stored_np(wp.q), ko, vo, stored_np(wp.block_tables), stored_np(wp.context_lens),
                    stored_np(wp.query_start_loc), wp.scale, "f32")
    err = assert_matches_oracle(out, ref, "f32", "f32 vllm prefill")
    _say(f"f32 vLLM-layout prefill: max err {err:.2e}")
    # append step: every sequence's newest token is new
    w = make_custom(num_seqs=4, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="f32",
                    lens=[1, 17, 64, 300], seed=72, device="cuda", poison=True)
    B = 4
    n = stored_np(w.context_lens).astype(np.int64)
    tbl = stored_np(w.block_tables)
    slots = np.array([tbl[b, (n[b] - 1) // 16] * 16 + (n[b] - 1) % 16 for b in range(B)], dtype=np.int64)
    k_new, v_new = make_new_rows(B, 2, 128, "f32", 73, "cuda")
    kc, vc = to_vllm_layout(w.k_cache, w.v_cache)
    out = pk.decode_append(w.q, kc, vc, k_new, v_new, torch.from_numpy(slots).cuda(), w.block_tables,
                           (w.context_lens - 1).to(torch.int32), w.scale, partition_size=64)
    torch.cuda.synchronize()
    ko, vo = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(ko, vo, stored_np(k_new), stored_np(v_new), slots)
    assert np.array_equal(_bits(stored_np(kc)), _bits(O.pack_k_vllm(ko, "f32")))
    assert np.array_equal(_bits(stored_np(vc)), _bits(O.pack_v_vllm(vo)))
    ref = O.decode(stored_np(w.q), ko, vo, tbl, stored_np(w.context_lens), w.scale, "f32")
    err = assert_matches_oracle(out, ref, "f32", "f32 vllm append")
    _say(f"f32 vLLM-layout append step: caches bit-exact, max err {err:.2e}")
