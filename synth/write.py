"""Seeded inputs for a large paged KV write (the scatter on its own).

A prefill-sized write: S prompts of L new tokens each, written into a shared
pool of blocks handed out in a shuffled order (10% spare blocks), so every run
of bs consecutive tokens of a prompt lands in one physical block and the
blocks of a prompt are scattered over the pool.  Optional padding slots (-1)
are spread through the batch.  Values are N(0, 1) drawn in fp32 and rounded
to the cache dtype; caches start as N(0, 1) too, so a missed or misplaced row
shows.  Holds no arithmetic of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict

import torch

from .workloads import torch_dtype

__all__ = ["WriteConfig", "WRITE_CONFIGS", "WriteWorkload", "make_write", "make_write_chunks", "make_new_rows"]


@dataclass(frozen=True)
class WriteConfig:
    name: str
    dtype: str
    num_prompts: int
    prompt_len: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    pad_tokens: int = 0
    pool_slack: float = 0.10
    seed: int = 0


# 65,536 tokens with the Llama-3-8B attention shape (KVH 8, D 128, bs 16):
# 16 prompts of 4096 tokens, 2 KiB per K row and per V row (~537 MB moved).
WRITE_CONFIGS: Dict[str, WriteConfig] = {
    "write_65536_bf16": WriteConfig(name="write_65536_bf16", dtype="bf16", num_prompts=16, prompt_len=4096,
                                    num_kv_heads=8, head_dim=128, block_size=16, seed=6),
}


@dataclass
class WriteWorkload:
    cfg: WriteConfig
    k_cache: torch.Tensor      # [NB, bs, KVH, D]
    v_cache: torch.Tensor
    k_new: torch.Tensor        # [T, KVH, D]
    v_new: torch.Tensor
    slot_mapping: torch.Tensor  # [T] int64
    valid_tokens: int

    def bytes_moved(self) -> int:
        """K and V rows read from k/v and written into the caches, plus the
        slot array (8 B per token, padding included)."""
        c = self.cfg
        elem = 4 if c.dtype == "f32" else 2
        row = c.num_kv_heads * c.head_dim * elem
        return self.valid_tokens * row * 2 * 2 + 8 * self.slot_mapping.numel()


def make_write(cfg: WriteConfig, device="cpu", *, num_prompts: int | None = None,
               prompt_len: int | None = None) -> WriteWorkload:
    """Seeded inputs of ``cfg`` (``num_prompts`` / ``prompt_len`` override its
    sizes for small parity cases)."""
    device = torch.device(device)
    S = cfg.num_prompts if num_prompts is None else num_prompts
    L = cfg.prompt_len if prompt_len is None else prompt_len
    bs, KVH, D = cfg.block_size, cfg.num_kv_heads, cfg.head_dim
    gm = torch.Generator().manual_seed(5000 + cfg.seed)
    gv = torch.Generator(device=device).manual_seed(6000 + cfg.seed)
    dt = torch_dtype(cfg.dtype)
    per = -(-L // bs)
    live = S * per
    NB = live + max(1, int(math.ceil(live * cfg.pool_slack)))
    perm = torch.randperm(NB, generator=gm)[:live].view(S, per)
    pos = torch.arange(L)
    slots = (perm[:, pos // bs] * bs + (pos % bs)).reshape(-1)
    valid = slots.numel()
    if cfg.pad_tokens:
        T = valid + cfg.pad_tokens
        where = torch.randperm(T, generator=gm)[:cfg.pad_tokens]
        full = torch.empty(T, dtype=torch.int64)
        mask = torch.ones(T, dtype=torch.bool)
        mask[where] = False
        full[~mask] = -1
        full[mask] = slots
        slots = full
    T = slots.numel()
    rnd = lambda *s: torch.randn(s, generator=gv, device=device, dtype=torch.float32).to(dt)
    k_cache, v_cache = rnd(NB, bs, KVH, D), rnd(NB, bs, KVH, D)
    k_new, v_new = rnd(T, KVH, D), rnd(T, KVH, D)
    return WriteWorkload(cfg=cfg, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                         slot_mapping=slots.to(device), valid_tokens=valid)


def make_write_chunks(*, num_kv_heads: int, head_dim: int, block_size: int, dtype: str, cached, new,
                      pad_tokens: int = 0, seed: int = 0, device="cpu") -> WriteWorkload:
    """Chunked-prefill writes: sequence i already holds cached[i] tokens and
    writes new[i] more, so its run of slots starts at offset cached[i] % bs of
    a block and crosses block boundaries wherever the chunk does.  Blocks come
    from one shuffled pool (10% spare); ``pad_tokens`` slots of -1 are spread
    through the batch."""
    device = torch.device(device)
    bs, KVH, D = block_size, num_kv_heads, head_dim
    gm = torch.Generator().manual_seed(7000 + seed)
    gv = torch.Generator(device=device).manual_seed(8000 + seed)
    per = [-(-(c + n) // bs) for c, n in zip(cached, new)]
    live = sum(per)
    NB = live + max(1, int(math.ceil(live * 0.10)))
    perm = torch.randperm(NB, generator=gm)[:live]
    runs, at = [], 0
    for c, n, m in zip(cached, new, per):
        table = perm[at:at + m]
        at += m
        pos = torch.arange(c, c + n)
        runs.append(table[pos // bs] * bs + pos % bs)
    slots = torch.cat(runs) if runs else torch.empty(0, dtype=torch.int64)
    valid = slots.numel()
    if pad_tokens:
        T = valid + pad_tokens
        where = torch.randperm(T, generator=gm)[:pad_tokens]
        mask = torch.ones(T, dtype=torch.bool)
        mask[where] = False
        full = torch.full((T,), -1, dtype=torch.int64)
        full[mask] = slots
        slots = full
    T = slots.numel()
    dt = torch_dtype(dtype)
    rnd = lambda *s: torch.randn(s, generator=gv, device=device, dtype=torch.float32).to(dt)
    k_cache, v_cache = rnd(NB, bs, KVH, D), rnd(NB, bs, KVH, D)
    k_new, v_new = rnd(T, KVH, D), rnd(T, KVH, D)
    cfg = WriteConfig(name="chunks", dtype=dtype, num_prompts=len(new), prompt_len=max(new, default=0),
                      num_kv_heads=KVH, head_dim=D, block_size=bs, pad_tokens=pad_tokens, seed=seed)
    return WriteWorkload(cfg=cfg, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                         slot_mapping=slots.to(device), valid_tokens=valid)


def make_new_rows(num_seqs: int, num_kv_heads: int, head_dim: int, dtype: str, seed: int, device="cpu"):
    """One new token's K and V rows per sequence, [num_seqs, KVH, D] each:
    N(0, 1) drawn in fp32 on ``device`` and rounded to the cache dtype."""
    device = torch.device(device)
    g = torch.Generator(device=device).manual_seed(9000 + seed)
    dt = torch_dtype(dtype)
    k = torch.randn(num_seqs, num_kv_heads, head_dim, generator=g, device=device, dtype=torch.float32).to(dt)
    v = torch.randn(num_seqs, num_kv_heads, head_dim, generator=g, device=device, dtype=torch.float32).to(dt)
    return k, v
