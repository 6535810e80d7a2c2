"""Seeded synthetic inputs for the paged prefill (varlen, causal).

Like ``synth.workloads`` this holds none of the method's arithmetic: it draws
lengths and values, hands out physical blocks and lists the slots of the new
tokens.  A prefill step is: write the new tokens' K/V rows into their slots
(``write_kv``), then attend with their queries.

Each sequence b has ``cached[b]`` tokens already in the cache and ``new[b]``
new tokens (its chunk), so its context after the write is
``n_b = cached[b] + new[b]`` and its queries are rows
``query_start_loc[b] .. query_start_loc[b+1] - 1`` of the packed ``q``.
Conventions (layout, int64 slots, int32 tables with 99999 tails, N(0, 1)
values rounded to the cache dtype) are those of ``synth.workloads``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

from .workloads import TAIL_FILL, torch_dtype

__all__ = ["PrefillConfig", "PREFILL_CONFIGS", "PrefillWorkload", "make_prefill", "make_prefill_custom"]


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """``cached`` / ``new`` draw the per-sequence counts:
    ("uniform", lo, hi) integers in [lo, hi], or ("explicit", (c0, c1, ...))."""

    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    cached: tuple
    new: tuple
    pool_slack: float = 0.10
    seed: int = 0


PREFILL_CONFIGS = {
    # Chunked prefill on the Llama-3-8B attention shape (H=32, KVH=8, D=128,
    # bs=16): 8 sequences, each with U[0, 4096] tokens already cached and a new
    # chunk of U[512, 2048] tokens.
    "prefill_8b_bf16": PrefillConfig(
        name="prefill_8b_bf16", dtype="bf16", num_seqs=8, num_heads=32, num_kv_heads=8,
        head_dim=128, block_size=16, cached=("uniform", 0, 4096), new=("uniform", 512, 2048), seed=5),
}


@dataclasses.dataclass
class PrefillWorkload:
    cfg: PrefillConfig
    k_cache: torch.Tensor          # [NB, bs, KVH, D] state before the write
    v_cache: torch.Tensor
    q: torch.Tensor                # [T, H, D]
    k_new: torch.Tensor            # [T, KVH, D]
    v_new: torch.Tensor
    slot_mapping: torch.Tensor     # [T] int64
    block_tables: torch.Tensor     # [B, W] int32
    context_lens: torch.Tensor     # [B] int32 (after the write)
    query_start_loc: torch.Tensor  # [B + 1] int32
    scale: float
    max_query_len: int
    cached: list
    new: list

    def flops(self) -> int:
        """Multiply-adds x 2 of the two products over the causally visible
        (query, key) pairs: 4 D flops per pair and query head."""
        c = self.cfg
        pairs = 0
        for cb, nb in zip(self.cached, self.new):
            pairs += nb * cb + nb * (nb + 1) // 2
        return 4 * c.head_dim * c.num_heads * pairs


def _draw(spec, B, g) -> list:
    if spec[0] == "uniform":
        return torch.randint(int(spec[1]), int(spec[2]) + 1, (B,), generator=g).tolist()
    if spec[0] == "explicit":
        v = [int(x) for x in spec[1]]
        assert len(v) == B
        return v
    raise ValueError(spec[0])


def make_prefill(cfg: PrefillConfig, device="cpu", *, poison: bool = False) -> PrefillWorkload:
    """Seeded inputs of ``cfg``.  ``poison=True`` fills every cache row no
    sequence reads with NaN (the new tokens' rows are written before the
    attention, so they are live)."""
    device = torch.device(device)
    gm = torch.Generator().manual_seed(3000 + cfg.seed)
    gv = torch.Generator(device=device).manual_seed(4000 + cfg.seed)
    dt = torch_dtype(cfg.dtype)
    B, H, KVH, D, bs = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    assert H % KVH == 0
    cached = _draw(cfg.cached, B, gm)
    new = _draw(cfg.new, B, gm)
    lens = [c + x for c, x in zip(cached, new)]
    nblk = [-(-n // bs) for n in lens]
    W = max(1, max(nblk))
    live_blocks = sum(nblk)
    NB = live_blocks + max(1, int(math.ceil(live_blocks * cfg.pool_slack)))
    perm = iter(torch.randperm(NB, generator=gm).tolist())
    rows = [[next(perm) for _ in range(nb)] for nb in nblk]
    table = torch.tensor([r + [TAIL_FILL] * (W - len(r)) for r in rows], dtype=torch.int64)

    slots, qsl = [], [0]
    for b in range(B):
        for pos in range(cached[b], lens[b]):
            slots.append(rows[b][pos // bs] * bs + pos % bs)
        qsl.append(qsl[-1] + new[b])
    T = len(slots)

    k_cache = torch.randn((NB, bs, KVH, D), generator=gv, device=device, dtype=torch.float32).to(dt)
    v_cache = torch.randn((NB, bs, KVH, D), generator=gv, device=device, dtype=torch.float32).to(dt)
    q = torch.randn((T, H, D), generator=gv, device=device, dtype=torch.float32).to(dt)
    k_new = torch.randn((T, KVH, D), generator=gv, device=device, dtype=torch.float32).to(dt)
    v_new = torch.randn((T, KVH, D), generator=gv, device=device, dtype=torch.float32).to(dt)
    if poison:
        mask = torch.ones(NB * bs, dtype=torch.bool)
        for b in range(B):
            for j, blk in enumerate(rows[b]):
                cnt = min(bs, lens[b] - j * bs)
                mask[blk * bs: blk * bs + cnt] = False
        mask_d = mask.to(device)
        k_cache.view(NB * bs, KVH, D)[mask_d] = float("nan")
        v_cache.view(NB * bs, KVH, D)[mask_d] = float("nan")
    return PrefillWorkload(
        cfg=cfg, k_cache=k_cache, v_cache=v_cache, q=q, k_new=k_new, v_new=v_new,
        slot_mapping=torch.tensor(slots, dtype=torch.int64).to(device),
        block_tables=table.to(torch.int32).to(device),
        context_lens=torch.tensor(lens, dtype=torch.int32).to(device),
        query_start_loc=torch.tensor(qsl, dtype=torch.int32).to(device),
        scale=1.0 / math.sqrt(D), max_query_len=max(new) if new else 0, cached=cached, new=new)


def make_prefill_custom(*, num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                        cached: Sequence[int], new: Sequence[int], dtype: str = "bf16", seed: int = 0,
                        device="cpu", poison: bool = False) -> PrefillWorkload:
    cfg = PrefillConfig(name="custom", dtype=dtype, num_seqs=len(cached), num_heads=num_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                        cached=("explicit", tuple(cached)), new=("explicit", tuple(new)), seed=seed)
    return make_prefill(cfg, device, poison=poison)
