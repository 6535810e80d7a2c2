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
from synth import WRITE_CONFIGS, make_write, to_vllm_layout
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
