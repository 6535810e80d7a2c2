"""pa_decode_noalloc (decode with the library's static device scratch area, for
callers that cannot allocate) against pa_decode with its own workspace,
through the C ABI, on an MI355X.

The two run the same kernels with the same partition size, so their outputs
agree bit for bit; both are also held to the oracle at the usual tolerance.
Calls follow one another on one stream with different sizes (the second one
smaller, then a different dtype), so a call that depended on what an earlier
one left in the shared scratch area would show.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import make_custom
from tests.gpu_util import assert_matches_oracle, stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on a CPU-only machine)")
    pk.load_library()
    yield


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_call(w, dtype, P, what):
    B, H, _ = w.q.shape
    W = w.block_tables.shape[1]
    need = pk.workspace_bytes(B, H, W, w.k_cache, P)
    assert 0 < need <= pk.NOALLOC_SCRATCH_BYTES, (what, need)
    ref_out = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, partition_size=P)
    out = torch.full_like(w.q, float("nan"))
    pk.decode_noalloc(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, out=out,
                      partition_size=P)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_out)), f"{what}: pa_decode_noalloc differs from pa_decode"
    ref = O.decode(stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache), stored_np(w.block_tables),
                   stored_np(w.context_lens), w.scale, dtype)
    err = assert_matches_oracle(out, ref, dtype, what)
    _say(f"{what}: B={B} H={H} W={W} P={P}, scratch {need} B, bit-equal to pa_decode, max err {err:.2e}")


def test_noalloc_equals_decode_two_calls_then_smaller():
    # first call: 24 sequences of mixed lengths, 256-token partitions (up to 16 of them)
    lens1 = np.random.default_rng(11).integers(1, 4000, size=24).tolist()
    lens1[0], lens1[1] = 1, 4000
    w1 = make_custom(num_seqs=24, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, dtype="bf16",
                     lens=lens1, seed=41, device="cuda")
    _check_call(w1, "bf16", 256, "call 1 (bf16, 24 sequences)")
    # second call, smaller: 5 sequences, another geometry; the area still holds call 1's partials
    w2 = make_custom(num_seqs=5, num_heads=8, num_kv_heads=2, head_dim=64, block_size=8, dtype="bf16",
                     lens=[700, 1, 129, 64, 333], seed=42, device="cuda")
    _check_call(w2, "bf16", 64, "call 2 (bf16, 5 sequences)")
    # third call: fp32 (the vector-ALU partial kernel and the same merge)
    w3 = make_custom(num_seqs=3, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype="f32",
                     lens=[200, 17, 90], seed=43, device="cuda")
    _check_call(w3, "f32", 32, "call 3 (fp32, 3 sequences)")


def test_noalloc_one_partition_and_limits():
    """A call needing no scratch (one partition) works, and a call needing
    more than the static area is refused before any launch."""
    w = make_custom(num_seqs=3, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                    lens=[5, 17, 100], seed=44, device="cuda")
    out = torch.empty_like(w.q)
    pk.decode_noalloc(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale, out=out)
    torch.cuda.synchronize()
    ref_out = pk.decode(w.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_out))
    # 4096 sequences x 64 heads of 64-token partitions over 4096-entry tables: far past 32 MiB
    big_tables = torch.zeros(4096, 4096, dtype=torch.int32, device="cuda")
    big_q = torch.zeros(4096, 64, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(4096, dtype=torch.int32, device="cuda")
    assert pk.workspace_bytes(4096, 64, 4096, w.k_cache, 64) > pk.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pk.PaError) as e:
        pk.decode_noalloc(big_q, w.k_cache, w.v_cache, big_tables, lens, 0.1, out=torch.empty_like(big_q),
                          partition_size=64)
    assert e.value.status == -11
    _say("one-partition call equal to pa_decode; oversize call refused with PA_ERR_SCRATCH")
