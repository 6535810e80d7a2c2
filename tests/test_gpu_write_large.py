"""The paged KV write at a prefill-sized token count, held to the oracle bit
for bit over the whole cache: 65,536 tokens (16 prompts of 4096) with the
Llama-3-8B shape, exactly as the write benchmark launches it, and smaller
cuts of the same recipe with padding slots spread through the batch, in both
cache dtypes and both layouts."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import WRITE_CONFIGS, make_write, make_write_chunks, to_vllm_layout
from tests.gpu_util import stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[gpu-write] {msg}", flush=True)
    sys.stdout.flush()


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _check(w, what):
    kc, vc = w.k_cache.clone(), w.v_cache.clone()
    pk.write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping)
    torch.cuda.synchronize()
    ko, vo = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(ko, vo, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    assert np.array_equal(_bits(stored_np(kc)), _bits(ko)), f"{what}: K cache"
    assert np.array_equal(_bits(stored_np(vc)), _bits(vo)), f"{what}: V cache"
    _say(f"{what}: {w.slot_mapping.numel()} tokens, bit-exact")


def test_write_65536_tokens_full_size():
    _check(make_write(WRITE_CONFIGS["write_65536_bf16"], "cuda"), "write_65536_bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S,L,pad", [(3, 37, 5), (5, 300, 17), (1, 1, 1)])
def test_write_prompt_batches_with_padding(dtype, S, L, pad):
    cfg = dataclasses.replace(WRITE_CONFIGS["write_65536_bf16"], dtype=dtype, pad_tokens=pad, seed=S + L)
    _check(make_write(cfg, "cuda", num_prompts=S, prompt_len=L), f"{dtype} S={S} L={L} pad={pad}")


def test_write_65536_tokens_vllm_layout():
    w = make_write(WRITE_CONFIGS["write_65536_bf16"], "cuda")
    kp, vp = to_vllm_layout(w.k_cache, w.v_cache)
    pk.write_kv(kp, vp, w.k_new, w.v_new, w.slot_mapping)
    torch.cuda.synchronize()
    ko, vo = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    O.write_kv(ko, vo, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    assert np.array_equal(stored_np(kp), O.pack_k_vllm(ko, "bf16")), "K cache (vLLM layout)"
    assert np.array_equal(stored_np(vp), O.pack_v_vllm(vo)), "V cache (vLLM layout)"
    _say("write_65536_bf16 in the vLLM layout: bit-exact")


# (dtype, KVH, D, bs, cached, new, pad): chunks that start mid-block and cross
# block edges; rows of 8, 24, 80 and 128 16-byte groups (the kernel takes 32 per
# workgroup, so 24 and 80 leave partial slices); token counts off the 16-token tile.
CHUNK_CASES = [
    ("bf16", 8, 128, 16, [1933, 889, 0, 15], [190, 75, 33, 1], 7),
    ("bf16", 1, 64, 8, [3, 0, 61], [29, 8, 100], 3),
    ("bf16", 3, 64, 32, [31, 32, 5], [2, 97, 40], 0),
    ("bf16", 5, 128, 64, [63, 1000], [130, 11], 5),
    ("f32", 2, 128, 16, [7, 40, 0], [50, 9, 16], 4),
    ("f32", 3, 64, 8, [1, 2], [17, 31], 1),
    ("bf16", 2, 256, 16, [], [], 3),            # padding only
]


@pytest.mark.parametrize("case", CHUNK_CASES,
                         ids=lambda c: f"{c[0]}_KVH{c[1]}_D{c[2]}_bs{c[3]}_T{sum(c[5]) + c[6]}")
def test_write_chunks_vllm_layout(case):
    """Chunked-prefill writes into vLLM's layout, bit-exact over both whole
    caches against the oracle's write on the packed caches."""
    dtype, KVH, D, bs, cached, new, pad = case
    w = make_write_chunks(num_kv_heads=KVH, head_dim=D, block_size=bs, dtype=dtype, cached=cached, new=new,
                          pad_tokens=pad, seed=KVH * D + bs + pad, device="cuda")
    kp, vp = to_vllm_layout(w.k_cache, w.v_cache)
    pk.write_kv(kp, vp, w.k_new, w.v_new, w.slot_mapping)
    torch.cuda.synchronize()
    ko = O.pack_k_vllm(stored_np(w.k_cache), dtype)
    vo = O.pack_v_vllm(stored_np(w.v_cache))
    O.write_kv_vllm(ko, vo, stored_np(w.k_new), stored_np(w.v_new), stored_np(w.slot_mapping))
    assert np.array_equal(_bits(stored_np(kp)), _bits(ko)), "K cache (vLLM layout)"
    assert np.array_equal(_bits(stored_np(vp)), _bits(vo)), "V cache (vLLM layout)"
    _say(f"chunks {dtype} KVH{KVH} D{D} bs{bs}: {w.slot_mapping.numel()} tokens, bit-exact")
