"""Seeded workload generators: shapes, metadata validity and determinism (CPU)."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, SENTINEL, TAIL_FILL, make_custom, make_workload


def _check_metadata(w):
    c = w.cfg
    B, bs = c.num_seqs, c.block_size
    NB = w.num_blocks
    lens = w.context_lens.tolist()
    tbl = w.block_tables.to(torch.int64)
    assert w.block_tables.dtype == torch.int32 and w.context_lens.dtype == torch.int32
    assert w.slot_mapping.dtype == torch.int64
    assert w.k_cache.shape == (NB, bs, c.num_kv_heads, c.head_dim)
    assert w.q.shape == (B, c.num_heads, c.head_dim)
    used = []
    for b in range(B):
        nb = -(-lens[b] // bs)
        row = tbl[b]
        assert bool(((row[:nb] >= 0) & (row[:nb] < NB)).all())
        if c.tail == "fill":
            assert bool((row[nb:] == TAIL_FILL).all())
        elif c.tail == "garbage":
            assert bool((row[nb:] >= NB).all())
        used.extend(row[:nb].tolist())
    slots = w.slot_mapping.tolist()
    valid = [s for s in slots if s >= 0]
    assert len(set(valid)) == len(valid) and all(s < NB * bs for s in valid)
    pad = w.slot_mapping < 0
    if w.k_new.device.type != "meta":
        assert bool((w.k_new[pad] == SENTINEL).all()) and bool((w.v_new[pad] == SENTINEL).all())
    return used


def test_tiny_config_matches_description():
    w = make_workload(CONFIGS["tiny_f32"])
    used = _check_metadata(w)
    lens = w.context_lens.tolist()
    assert 1 in lens and 192 in lens and all(1 <= n <= 200 for n in lens)
    assert w.num_blocks == 64 and len(set(used)) == len(used)
    slots = w.slot_mapping.tolist()
    assert len(slots) == 6 and slots.count(-1) == 1
    # 4 newest-token slots live in the tables; one slot lives in an unused block
    tbl = w.block_tables.to(torch.int64)
    owners = [s // 16 for s in slots if s >= 0]
    assert sum(1 for o in owners if o in set(used)) == 4
    assert sum(1 for o in owners if o in set(w.unused_blocks.tolist())) == 1


@pytest.mark.parametrize("name", ["llama3_8b_bf16", "big_batch_bf16", "prefix_shared_bf16"])
def test_metadata_of_big_configs(name):
    cfg = CONFIGS[name]
    w = make_workload(cfg, values=False)
    used = _check_metadata(w)
    if cfg.ctx[0] == "prefix":
        tbl = w.block_tables.to(torch.int64)
        assert bool((tbl[:, :128] == tbl[0, :128]).all())
        private = [x for x in used if x not in set(tbl[0, :128].tolist())]
        assert len(set(private)) == len(private)
    else:
        assert len(set(used)) == len(used)
    if name == "big_batch_bf16":
        s = w.slot_mapping.tolist()
        assert len(s) == 320 and s[256:] == [-1] * 64 and min(s[:256]) >= 0
        lens = w.context_lens.tolist()
        assert min(lens) >= 128 and max(lens) <= 8192


def test_deterministic_and_poison():
    a = make_custom(num_seqs=3, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                    lens=[1, 4, 9], seed=5, pad_tokens=2, tail="poison", poison=True)
    b = make_custom(num_seqs=3, num_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                    lens=[1, 4, 9], seed=5, pad_tokens=2, tail="poison", poison=True)
    assert torch.equal(a.q, b.q) and torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.k_cache.isnan(), b.k_cache.isnan())
    flat = a.k_cache.reshape(-1, 2, 8)
    live = torch.zeros(flat.shape[0], dtype=torch.bool)
    live[a.live_slots] = True
    assert bool(flat[live].isfinite().all()) and bool(flat[~live].isnan().all())
    # poison tails point at NaN blocks that exist
    tbl = a.block_tables.to(torch.int64)
    assert int(tbl.max()) < a.num_blocks


def test_write_workload_recipe():
    """Prompt runs of bs tokens share one block, slots are distinct and inside
    the pool, padding slots are -1, and the full-size recipe moves ~537 MB."""
    import dataclasses

    from synth import WRITE_CONFIGS, make_write
    base = WRITE_CONFIGS["write_65536_bf16"]
    cfg = dataclasses.replace(base, pad_tokens=7)
    w = make_write(cfg, num_prompts=4, prompt_len=50)
    s = w.slot_mapping.tolist()
    assert len(s) == 4 * 50 + 7 and s.count(-1) == 7 and w.valid_tokens == 200
    valid = [x for x in s if x >= 0]
    assert len(set(valid)) == len(valid) and max(valid) < w.k_cache.shape[0] * cfg.block_size
    for p in range(4):
        run = valid[p * 50:(p + 1) * 50]
        for t in range(50):
            assert run[t] % 16 == t % 16 and run[t] // 16 == run[t - t % 16] // 16
    S, L = base.num_prompts, base.prompt_len
    assert S * L == 65536
    row = base.num_kv_heads * base.head_dim * 2
    assert S * L * row * 4 + 8 * S * L == 537_395_200
