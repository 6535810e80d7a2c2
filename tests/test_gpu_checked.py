"""Checked mode on an MI355X: pa_check_write / pa_check_decode /
pa_check_prefill flag exactly the broken preconditions, through the C ABI.

Every bad input here is one the hot-path kernels stay memory-safe on, and
the check kernels themselves only read what those kernels read.  Each case
is also given to the oracle, which refuses exactly the inputs that break a
precondition (it raises OracleError): a flag must be set if and only if the
oracle refuses.  Cases follow "P09 · Paged KV 写入 + decode attention":
padding slots (-1 and other negative values) are not violations (题面速览);
a slot past the cache, or two tokens with one slot, are; a garbage table
entry the sequence uses is, one in the unused tail is not (细节, 易错点).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import CONFIGS, make_custom, make_prefill_custom, make_workload, stored_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[checked] {msg}", flush=True)
    sys.stdout.flush()


def _flags_write(slots, k_cache):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.check_write(slots, k_cache, err)
    torch.cuda.synchronize()
    return int(err.item())


def _flags_decode(tables, lens, k_cache):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.check_decode(tables, lens, k_cache, err)
    torch.cuda.synchronize()
    return int(err.item())


def _oracle_refuses(fn, *a):
    try:
        fn(*a)
        return False
    except O.OracleError:
        return True


def _oracle_write_refuses(w, slots):
    ko, vo = stored_np(w.k_cache).copy(), stored_np(w.v_cache).copy()
    T = slots.numel()
    k = np.zeros((T, *ko.shape[2:]), dtype=ko.dtype)
    return _oracle_refuses(O.write_kv, ko, vo, k, k.copy(), stored_np(slots))


def _oracle_decode_refuses(w, tables, lens):
    return _oracle_refuses(O.decode, stored_np(w.q), stored_np(w.k_cache), stored_np(w.v_cache), stored_np(tables),
                           stored_np(lens), w.scale, w.cfg.dtype)


@pytest.mark.parametrize("name", ["tiny_f32", "llama3_8b_bf16", "big_batch_bf16"])
def test_workloads_pass_the_checks(name):
    """The workloads' own inputs (padding slots, 99999 or garbage table tails)
    break no precondition."""
    w = make_workload(CONFIGS[name], "cuda")
    assert _flags_write(w.slot_mapping, w.k_cache) == 0
    assert _flags_decode(w.block_tables, w.context_lens, w.k_cache) == 0
    _say(f"{name}: no flags")


def _small():
    return make_custom(num_seqs=5, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, dtype="f32",
                       lens=[1, 16, 40, 200, 33], pad_tokens=2, seed=61, device="cuda")


def test_write_flags():
    w = _small()
    NB, bs = w.k_cache.shape[0], w.k_cache.shape[1]
    base = w.slot_mapping.clone()
    valid = torch.nonzero(base >= 0).flatten()
    cases = {}
    s = base.clone()
    s[int(valid[0])] = NB * bs                        # one past the last slot
    cases["past the cache"] = (s, pk.CHECK_SLOT_RANGE)
    s = base.clone()
    s[int(valid[1])] = 2 ** 40                        # far past it (int64 slots)
    cases["far past the cache"] = (s, pk.CHECK_SLOT_RANGE)
    s = base.clone()
    s[int(valid[2])] = s[int(valid[3])]
    cases["duplicate"] = (s, pk.CHECK_SLOT_DUPLICATE)
    s = base.clone()
    s[int(valid[0])] = NB * bs + 3
    s[int(valid[2])] = s[int(valid[3])]
    cases["both"] = (s, pk.CHECK_SLOT_RANGE | pk.CHECK_SLOT_DUPLICATE)
    s = base.clone()
    s[int(valid[0])] = -7                             # any negative slot is padding
    s[int(valid[1])] = -1
    cases["padding"] = (s, 0)
    cases["last slot"] = (torch.tensor([NB * bs - 1, 0, -1], dtype=torch.int64, device="cuda"), 0)
    for what, (slots, want) in cases.items():
        got = _flags_write(slots, w.k_cache)
        refuses = _oracle_write_refuses(w, slots)
        assert got == want, (what, got, want)
        assert refuses == (want != 0), (what, refuses)
        _say(f"write, {what}: flags {got:#x}, oracle {'refuses' if refuses else 'accepts'}")


def test_write_duplicates_at_scale():
    """65,536 distinct slots pass; one repeated pair among them is found."""
    NB, bs = 8192, 16
    kc = torch.zeros((NB, bs, 1, 64), dtype=torch.bfloat16, device="cuda")
    perm = torch.randperm(NB * bs, generator=torch.Generator().manual_seed(5))[:65536].to("cuda")
    assert _flags_write(perm, kc) == 0
    perm[40000] = perm[123]
    assert _flags_write(perm, kc) == pk.CHECK_SLOT_DUPLICATE


def test_decode_flags():
    w = _small()
    NB, bs = w.k_cache.shape[0], w.k_cache.shape[1]
    W = w.block_tables.shape[1]
    lens = w.context_lens.clone()
    n3 = int(lens[3])
    cases = {}
    t = w.block_tables.clone()
    t[3, (n3 - 1) // bs] = 99999                      # the last block sequence 3 uses
    cases["garbage entry in use"] = (t, lens, pk.CHECK_TABLE_RANGE)
    t = w.block_tables.clone()
    t[2, 0] = -1
    cases["negative entry in use"] = (t, lens, pk.CHECK_TABLE_RANGE)
    t = w.block_tables.clone()
    t[3, -(-n3 // bs):] = 99999                       # the unused tail: never read
    cases["garbage tail"] = (t, lens, 0)
    t = w.block_tables.clone()
    t[1, 1:] = NB                                     # sequence 1 (16 tokens) uses entry 0 only
    cases["tail past a full block"] = (t, lens, 0)
    full = w.block_tables.clone()
    full[0] = torch.arange(W, dtype=torch.int32, device="cuda") % NB   # a row with every entry in the pool
    l2 = lens.clone()
    l2[0] = W * bs + 1                                # clamped to W * bs: every entry of the row is read
    cases["length past the table"] = (full, l2, pk.CHECK_CONTEXT_RANGE)
    cases["length past the table, garbage tail"] = (w.block_tables, l2,
                                                    pk.CHECK_CONTEXT_RANGE | pk.CHECK_TABLE_RANGE)
    l2 = lens.clone()
    l2[4] = -1
    cases["negative length"] = (w.block_tables, l2, pk.CHECK_CONTEXT_RANGE)
    l2 = lens.clone()
    l2[0] = W * bs                                    # the whole table: allowed
    cases["whole table"] = (full, l2, 0)
    for what, (tables, ln, want) in cases.items():
        got = _flags_decode(tables, ln, w.k_cache)
        refuses = _oracle_decode_refuses(w, tables, ln)
        assert got == want, (what, got, want)
        assert refuses == (want != 0), (what, refuses)
        _say(f"decode, {what}: flags {got:#x}, oracle {'refuses' if refuses else 'accepts'}")


def test_prefill_flags():
    w = make_prefill_custom(num_heads=8, num_kv_heads=2, head_dim=64, block_size=16, cached=[0, 30, 5],
                            new=[20, 3, 40], dtype="bf16", seed=62, device="cuda")
    T = w.q.shape[0]

    def flags(qsl, lens=None):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        pk.check_prefill(w.block_tables, w.context_lens if lens is None else lens, qsl, T, w.k_cache, err)
        torch.cuda.synchronize()
        return int(err.item())

    def refuses(qsl, lens=None):
        ko, vo = stored_np(w.k_cache), stored_np(w.v_cache)
        return _oracle_refuses(O.prefill, stored_np(w.q), ko, vo, stored_np(w.block_tables),
                               stored_np(w.context_lens if lens is None else lens), stored_np(qsl), w.scale, "bf16")

    qsl = w.query_start_loc
    assert flags(qsl) == 0 and not refuses(qsl)
    bad = qsl.clone()
    a, b = int(bad[1]), int(bad[2])
    bad[1], bad[2] = b, a                             # decreasing
    assert flags(bad) == pk.CHECK_QUERY_RANGE and refuses(bad)
    bad = qsl.clone()
    bad[-1] = T - 1                                   # does not end at T
    assert flags(bad) == pk.CHECK_QUERY_RANGE and refuses(bad)
    lens = w.context_lens.clone()
    lens[2] = 30                                      # 40 new queries, 30 tokens
    assert flags(qsl, lens) == pk.CHECK_QUERY_RANGE and refuses(qsl, lens)
    _say("prefill: query_start_loc order and end, and L_b > n_b, flagged as the oracle refuses them")
