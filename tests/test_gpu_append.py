"""pa_decode_append on an MI355X, held to the oracle: one decode step whose
new token per sequence is written into the cache and folded into the softmax
by the merge kernel (read from k_new / v_new, not the cache).

Expected values: the oracle's write_kv of the new rows, then its decode with
context = cached + 1 ("P09 · Paged KV 写入 + decode attention", 题面速览 and the
decode shape trace).  The caches are compared bit for bit; the outputs within
the dtype's tolerance.  Cases: fresh sequences (cached 0), cached lengths on
and off partition and block edges, sequences with no new token (slot -1),
padding-only sequences (cached 0 and slot -1), both layouts, both dtypes,
merges that take several rounds, and the full-size Llama-3-8B-shape and
long-context steps (every sequence).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import CONFIGS, make_custom, make_new_rows, make_workload, to_vllm_layout
from tests.gpu_util import assert_matches_oracle, oracle_per_sequence, stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[gpu-append] {msg}", flush=True)
    sys.stdout.flush()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _step(w, no_new=(), vllm=False, partition_size=0):
    """Run the append step on w: sequence b's newest token (position n_b - 1)
    is the new one unless b is in no_new (then all n_b tokens are cached and
    its slot is -1).  Returns (out, caches after, oracle out, oracle caches)."""
    B = w.q.shape[0]
    n = stored_np(w.context_lens).astype(np.int64)
    tbl = stored_np(w.block_tables)
    bs = w.k_cache.shape[1]
    has = np.array([b not in no_new and n[b] > 0 for b in range(B)])
    cached = np.where(has, n - 1, n)
    slots = np.array([tbl[b, (n[b] - 1) // bs] * bs + (n[b] - 1) % bs if has[b] else -1 for b in range(B)],
                     dtype=np.int64)
    KVH, D = w.k_cache.shape[2], w.k_cache.shape[3]
    k_new, v_new = make_new_rows(B, KVH, D, w.cfg.dtype, B * 131 + int(n.sum()) % 1000, w.q.device)
    # oracle: write the new rows, then decode over cached + new
    ko, vo = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(ko, vo, stored_np(k_new), stored_np(v_new), slots)
    ref = O.decode(stored_np(w.q), ko, vo, tbl, (cached + has).astype(np.int32), w.scale, w.cfg.dtype)
    kc, vc = (to_vllm_layout(w.k_cache, w.v_cache) if vllm else (w.k_cache.clone(), w.v_cache.clone()))
    out = pk.decode_append(w.q, kc, vc, k_new, v_new, torch.from_numpy(slots).to(w.q.device), w.block_tables,
                           torch.from_numpy(cached.astype(np.int32)).to(w.q.device), w.scale,
                           partition_size=partition_size)
    torch.cuda.synchronize()
    if vllm:
        ko, vo = O.pack_k_vllm(ko, w.cfg.dtype), O.pack_v_vllm(vo)
    assert np.array_equal(_bits(stored_np(kc)), _bits(ko)), "K cache"
    assert np.array_equal(_bits(stored_np(vc)), _bits(vo)), "V cache"
    return out, ref


# (dtype, H, KVH, D, bs, P, lengths incl. the new token, sequences without a new token)
CASES = [
    ("bf16", 8, 2, 128, 16, 64, [1, 2, 16, 17, 64, 65, 129, 300, 1000], (3,)),
    ("bf16", 32, 8, 128, 16, 0, [1, 33, 500, 2048, 4000], ()),
    ("bf16", 16, 2, 64, 8, 32, [1, 9, 31, 32, 33, 250], (5,)),
    ("bf16", 4, 2, 256, 32, 0, [7, 64, 65, 700], (0,)),
    ("f32", 8, 2, 64, 16, 32, [1, 16, 40, 200], (2,)),
    ("f32", 4, 4, 128, 16, 0, [3, 77], ()),
    # more partitions than the merge folds in one round (32 for head_dim 128, 16 for 256, 64 for 64):
    # 63, 44 and 75 partitions
    ("bf16", 8, 2, 128, 16, 16, [1000, 17, 520, 1], (2,)),
    ("bf16", 4, 2, 256, 16, 16, [700, 300, 16], ()),
    ("bf16", 8, 4, 64, 8, 8, [600, 9, 64], ()),
]


@pytest.mark.parametrize("vllm", [False, True], ids=["p09", "vllm"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_H{c[1]}_KVH{c[2]}_D{c[3]}_bs{c[4]}_P{c[5]}")
def test_append_matches_write_then_decode(case, vllm):
    """Poisoned caches (every row that no sequence reads holds NaN), in both
    layouts."""
    dtype, H, KVH, D, bs, P, lens, no_new = case
    w = make_custom(num_seqs=len(lens), num_heads=H, num_kv_heads=KVH, head_dim=D, block_size=bs, dtype=dtype,
                    lens=lens, seed=H + D + bs, device="cuda", poison=True)
    out, ref = _step(w, no_new, vllm=vllm, partition_size=P)
    err = assert_matches_oracle(out, ref, dtype, f"append {dtype} H{H} D{D} bs{bs} P{P}")
    _say(f"{dtype} H{H} KVH{KVH} D{D} bs{bs} P{P} {'vllm' if vllm else 'p09'}: max err {err:.2e}")


@pytest.mark.parametrize("vllm", [False, True], ids=["p09", "vllm"])
def test_append_beyond_persistent_list(vllm):
    """4,100 sequences: more than the bf16 persistent kernel's list holds
    (4,096), so the partials run in the grid form (the P09 layout's
    matrix-core grid kernel, the vLLM layout's own)."""
    rng = np.random.default_rng(4100)
    lens = [int(x) for x in rng.integers(1, 40, size=4100)]
    w = make_custom(num_seqs=len(lens), num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype="bf16",
                    lens=lens, seed=4100, device="cuda")
    out, ref = _step(w, (7, 4099), vllm=vllm)
    err = assert_matches_oracle(out, ref, "bf16", "4,100 sequences")
    _say(f"4,100 sequences ({'vllm' if vllm else 'p09'}): caches bit-exact, max err {err:.2e}")


def test_append_padding_sequences_and_vllm_layout():
    """Sequences of length 0 with slot -1 (graph padding) give zeros and write
    nothing; the same batch in vLLM's layout."""
    lens = [0, 5, 0, 130, 64, 0]
    w = make_custom(num_seqs=len(lens), num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                    lens=lens, seed=77, device="cuda")
    out, ref = _step(w)
    assert_matches_oracle(out, ref, "bf16", "padding")
    assert not bool(out[0].float().abs().any()) and not bool(out[2].float().abs().any())
    out, ref = _step(w, vllm=True, partition_size=64)
    assert_matches_oracle(out, ref, "bf16", "vLLM layout")


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "long_ctx_bf16"])
def test_append_full_size_step(name):
    """The full-size steps the benchmark times as one pa_decode_append call
    (Llama-3-8B shape: 64 sequences up to 4096 tokens; long context: 8
    sequences of 32k-131k tokens, up to 128 partitions, so the merge folds
    several rounds) at the automatic partition size: caches bit for bit
    against write_kv, and every sequence against the oracle."""
    w = make_workload(CONFIGS[name], "cuda")
    err = _step_full(w)
    _say(f"{name} append step: caches bit-exact, all {w.q.shape[0]} sequences within tolerance, "
         f"max err {err:.2e}")


def _step_full(w):
    B = w.q.shape[0]
    n = stored_np(w.context_lens).astype(np.int64)
    tbl = stored_np(w.block_tables)
    bs = w.k_cache.shape[1]
    slots = torch.from_numpy(np.array([tbl[b, (n[b] - 1) // bs] * bs + (n[b] - 1) % bs for b in range(B)],
                                      dtype=np.int64)).to(w.q.device)
    cached = (w.context_lens - 1).to(torch.int32)
    KVH, D = w.k_cache.shape[2], w.k_cache.shape[3]
    k_new, v_new = make_new_rows(B, KVH, D, "bf16", 3, w.q.device)
    k1, v1 = w.k_cache.clone(), w.v_cache.clone()
    pk.write_kv(k1, v1, k_new, v_new, slots)
    k2, v2 = w.k_cache.clone(), w.v_cache.clone()
    out = pk.decode_append(w.q, k2, v2, k_new, v_new, slots, w.block_tables, cached, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2), "caches"
    del k2, v2
    kc, vc = stored_np(k1), stored_np(v1)
    q, lens = stored_np(w.q), stored_np(w.context_lens)
    ref = oracle_per_sequence(lambda b0, b1: O.decode(q[b0:b1], kc, vc, tbl[b0:b1], lens[b0:b1], w.scale, "bf16"), B)
    return assert_matches_oracle(out, ref, "bf16", "append step")
