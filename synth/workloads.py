"""Seeded synthetic inputs for the paged KV write and paged decode attention.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds none of the method's arithmetic: it draws random values,
sizes a block pool, hands out physical blocks (what a block allocator would do
before the kernels run) and records which cache slots hold live tokens. It
never performs the write, the gather or the attention itself.

Conventions follow the problem statement of "P09 · Paged KV 写入 + decode
attention" (kuanzhou.online, section 题面速览):

* cache layout ``[num_blocks, block_size, num_kv_heads, head_dim]``;
* ``slot_mapping [T]`` int64, ``-1`` marks a padding token (CUDA-graph padded
  batches, same section);
* ``block_tables [B, W]`` int32, a padded rectangle whose tail entries are
  garbage (same page, section 细节);
* ``context_lens [B]`` int32; in decode the newest token is already written
  and is part of its own context (same page, section 细节).

Values are N(0, 1) drawn in fp32 and rounded to the cache dtype by torch's
round-to-nearest-even cast; padding rows carry the sentinel 9.0 (invariant I1
of the same page, section 不变量).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import torch

__all__ = [
    "Config",
    "CONFIGS",
    "CONFIG_ORDER",
    "Workload",
    "make_workload",
    "make_custom",
    "torch_dtype",
    "bits_view",
    "stored_np",
    "SENTINEL",
    "TAIL_FILL",
    "to_vllm_layout",
]

SENTINEL = 9.0          # value carried by padding rows (slot = -1)
TAIL_FILL = 99999       # garbage written into unused block-table entries


@dataclasses.dataclass(frozen=True)
class Config:
    """One benchmark / parity workload.

    ``ctx`` selects how context lengths are drawn:
      ("uniform", lo, hi)        integers uniform in [lo, hi]
      ("loguniform", lo, hi)     round(exp(U(log lo, log hi)))
      ("prefix", P, lo, hi)      P shared prefix tokens + uniform[lo, hi] suffix
      ("explicit", (n0, n1, …))  given lengths
    """

    name: str
    dtype: str                      # "f32" | "bf16"
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx: tuple
    forced_lens: tuple = ()         # lengths placed in the first sequences
    num_blocks: Optional[int] = None  # fixed pool size; default live + slack
    pool_slack: float = 0.10
    tail: str = "fill"              # "fill" (99999) | "garbage" | "poison"
    write: str = "newest"           # "newest" | "newest+extra"
    pad_tokens: int = 0             # trailing padding slots (-1)
    shuffle_write: bool = False
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def max_len(self) -> int:
        kind = self.ctx[0]
        if kind in ("uniform", "loguniform"):
            return int(self.ctx[2])
        if kind == "prefix":
            return int(self.ctx[1]) + int(self.ctx[3])
        if kind == "explicit":
            return int(max(self.ctx[1]))
        raise ValueError(kind)

    def table_width(self) -> int:
        return max(1, -(-self.max_len() // self.block_size))


# The five workloads.  Seeds are the config index.
CONFIGS = {
    # Tiny fp32: B=4, H=8, KVH=2, D=64, bs=16, lengths U[1,200] with one n=1 and
    # one multiple of 16; a fixed 64-block pool; T=6 writes (4 newest tokens, one
    # token in an otherwise unused block, one padding slot), shuffled.
    "tiny_f32": Config(
        name="tiny_f32", dtype="f32", num_seqs=4, num_heads=8, num_kv_heads=2,
        head_dim=64, block_size=16, ctx=("uniform", 1, 200), forced_lens=(1, 192),
        num_blocks=64, tail="fill", write="newest+extra", pad_tokens=1,
        shuffle_write=True, seed=0),
    # Llama-3-8B attention shape: B=64, H=32, KVH=8, D=128, bs=16, U[1,4096].
    "llama3_8b_bf16": Config(
        name="llama3_8b_bf16", dtype="bf16", num_seqs=64, num_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16, ctx=("uniform", 1, 4096),
        tail="fill", seed=1),
    # Long context, split-KV: B=8, lengths U[32768,131072], garbage tails.
    "long_ctx_bf16": Config(
        name="long_ctx_bf16", dtype="bf16", num_seqs=8, num_heads=32,
        num_kv_heads=8, head_dim=128, block_size=16,
        ctx=("uniform", 32768, 131072), tail="garbage", seed=2),
    # Large padded batch: B=256, H=64, KVH=8, bs=32, log-uniform[128,8192],
    # 320 written slots of which the last 64 are padding.
    "big_batch_bf16": Config(
        name="big_batch_bf16", dtype="bf16", num_seqs=256, num_heads=64,
        num_kv_heads=8, head_dim=128, block_size=32,
        ctx=("loguniform", 128, 8192), tail="fill", pad_tokens=64, seed=3),
    # Prefix-shared blocks: every table starts with the same 128 physical blocks
    # (a 2048-token prefix), then a private shuffled suffix of U[1,2048] tokens.
    "prefix_shared_bf16": Config(
        name="prefix_shared_bf16", dtype="bf16", num_seqs=128, num_heads=16,
        num_kv_heads=4, head_dim=256, block_size=16,
        ctx=("prefix", 2048, 1, 2048), tail="fill", seed=4),
}
CONFIG_ORDER = ["tiny_f32", "llama3_8b_bf16", "long_ctx_bf16", "big_batch_bf16",
                "prefix_shared_bf16"]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def bits_view(t: torch.Tensor) -> torch.Tensor:
    """Same storage reinterpreted as unsigned-width integers (for bit compares)."""
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    raise TypeError(t.dtype)


def stored_np(t: torch.Tensor):
    """The stored values of ``t`` on the host, unconverted: float32 as is,
    bfloat16 as its 16-bit patterns (which the oracle widens exactly)."""
    import numpy as np

    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclasses.dataclass
class Workload:
    cfg: Config
    k_cache: torch.Tensor         # [NB, bs, KVH, D]  (state before the write)
    v_cache: torch.Tensor
    q: torch.Tensor               # [B, H, D]
    k_new: torch.Tensor           # [T, KVH, D]
    v_new: torch.Tensor
    slot_mapping: torch.Tensor    # [T] int64, -1 = padding
    block_tables: torch.Tensor    # [B, W] int32
    context_lens: torch.Tensor    # [B] int32
    scale: float
    live_slots: torch.Tensor      # [L] int64: every slot some sequence reads (CPU)
    unused_blocks: torch.Tensor   # [U] int64: physical blocks no table references (CPU)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of K and V rows the decode has to read (sum of n_b rows)."""
        c = self.cfg
        elem = 4 if c.dtype == "f32" else 2
        return int(self.context_lens.to(torch.int64).sum()) * 2 * c.num_kv_heads * c.head_dim * elem

    def kv_unique_bytes(self) -> int:
        """Bytes of the distinct K and V rows the decode reads: a block that
        several tables share counts once (equal to kv_bytes() without
        sharing).  The least the decode must fetch from HBM."""
        c = self.cfg
        elem = 4 if c.dtype == "f32" else 2
        return int(self.live_slots.numel()) * 2 * c.num_kv_heads * c.head_dim * elem


def _draw_lengths(cfg: Config, g: torch.Generator) -> list[int]:
    B = cfg.num_seqs
    kind = cfg.ctx[0]
    if kind == "uniform":
        lo, hi = int(cfg.ctx[1]), int(cfg.ctx[2])
        lens = torch.randint(lo, hi + 1, (B,), generator=g).tolist()
    elif kind == "loguniform":
        lo, hi = float(cfg.ctx[1]), float(cfg.ctx[2])
        u = torch.rand((B,), generator=g, dtype=torch.float64)
        lens = [int(min(hi, max(lo, round(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo)))))))
                for x in u.tolist()]
    elif kind == "prefix":
        p, lo, hi = int(cfg.ctx[1]), int(cfg.ctx[2]), int(cfg.ctx[3])
        lens = [p + x for x in torch.randint(lo, hi + 1, (B,), generator=g).tolist()]
    elif kind == "explicit":
        lens = [int(x) for x in cfg.ctx[1]]
        assert len(lens) == B
    else:
        raise ValueError(kind)
    for i, n in enumerate(cfg.forced_lens):
        lens[i] = int(n)
    return lens


def _randn(shape, dtype: torch.dtype, g: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)


def make_workload(cfg: Config, device="cpu", *, poison: bool = False,
                  lens: Optional[Sequence[int]] = None, values: bool = True) -> Workload:
    """Build the seeded inputs of ``cfg`` on ``device``.

    Metadata (lengths, block assignment, slots) is drawn on the CPU; the big
    value tensors are drawn with a generator on ``device`` (so a GPU run does not
    have to push gigabytes through PCIe).  ``poison=True`` fills every cache row
    that no sequence reads with NaN, and makes ``tail == "poison"`` tables point
    their tails at NaN-filled blocks.  ``values=False`` builds the metadata only
    (value tensors live on the ``meta`` device: shapes without storage).
    """
    device = torch.device(device)
    gm = torch.Generator().manual_seed(1000 + cfg.seed)
    gv = torch.Generator(device=device).manual_seed(2000 + cfg.seed)
    dt = torch_dtype(cfg.dtype)
    B, H, KVH, D, bs = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.block_size
    assert H % KVH == 0
    W = cfg.table_width()
    lens = list(lens) if lens is not None else _draw_lengths(cfg, gm)
    assert len(lens) == B and all(0 <= n <= W * bs for n in lens)

    nblk = [-(-n // bs) for n in lens]
    if cfg.ctx[0] == "prefix":
        shared = int(cfg.ctx[1]) // bs
        assert int(cfg.ctx[1]) % bs == 0
        private = [nb - shared for nb in nblk]
        live_blocks = shared + sum(private)
    else:
        shared = 0
        private = nblk
        live_blocks = sum(nblk)
    extra_needed = 1 if cfg.write == "newest+extra" else 0
    if cfg.num_blocks is not None:
        NB = cfg.num_blocks
    else:
        NB = live_blocks + max(1 + extra_needed, int(math.ceil(live_blocks * cfg.pool_slack)))
    assert NB >= live_blocks + extra_needed, "pool too small"

    perm = torch.randperm(NB, generator=gm).tolist()
    it = iter(perm)
    shared_ids = [next(it) for _ in range(shared)]
    table = torch.empty((B, W), dtype=torch.int64)
    rows = []
    for b in range(B):
        ids = shared_ids + [next(it) for _ in range(private[b])]
        rows.append(ids)
    unused = list(it)                      # blocks no table references
    extra_block = unused[0] if extra_needed else None

    # Tail entries.
    for b in range(B):
        ids = rows[b]
        tail_n = W - len(ids)
        if cfg.tail == "fill":
            tail = [TAIL_FILL] * tail_n
        elif cfg.tail == "garbage":
            tail = torch.randint(NB, 2**31 - 1, (tail_n,), generator=gm).tolist()
        elif cfg.tail == "poison":
            cand = unused[1:] if extra_needed else unused
            assert cand, "poison tails need at least one spare block"
            tail = [cand[(b + j) % len(cand)] for j in range(tail_n)]
        else:
            raise ValueError(cfg.tail)
        table[b] = torch.tensor(ids + tail, dtype=torch.int64)

    # Slots of the newest token of each sequence (position n-1), the allocator's
    # (block, offset) -> flat slot numbering of the cache.
    slots = []
    for b in range(B):
        n = lens[b]
        if n == 0:
            continue
        pos = n - 1
        slots.append(rows[b][pos // bs] * bs + pos % bs)
    if extra_needed:
        off = int(torch.randint(0, bs, (1,), generator=gm))
        slots.append(extra_block * bs + off)
    n_real = len(slots)
    slots = slots + [-1] * cfg.pad_tokens
    T = len(slots)
    slot_t = torch.tensor(slots, dtype=torch.int64)
    if cfg.shuffle_write:
        slot_t = slot_t[torch.randperm(T, generator=gm)]

    # Live slots: every (block, offset) some sequence reads.
    live = []
    for b in range(B):
        n = lens[b]
        for j, blk in enumerate(rows[b]):
            cnt = min(bs, n - j * bs)
            live.extend(range(blk * bs, blk * bs + cnt))
    live_t = torch.unique(torch.tensor(live, dtype=torch.int64)) if live else torch.empty(0, dtype=torch.int64)

    # Values.
    if not values:
        meta = lambda shape: torch.empty(shape, dtype=dt, device="meta")
        return Workload(
            cfg=cfg, k_cache=meta((NB, bs, KVH, D)), v_cache=meta((NB, bs, KVH, D)),
            q=meta((B, H, D)), k_new=meta((T, KVH, D)), v_new=meta((T, KVH, D)),
            slot_mapping=slot_t, block_tables=table.to(torch.int32),
            context_lens=torch.tensor(lens, dtype=torch.int32), scale=1.0 / math.sqrt(D),
            live_slots=live_t, unused_blocks=torch.tensor(unused, dtype=torch.int64))
    k_cache = _randn((NB, bs, KVH, D), dt, gv, device)
    v_cache = _randn((NB, bs, KVH, D), dt, gv, device)
    q = _randn((B, H, D), dt, gv, device)
    k_new = _randn((T, KVH, D), dt, gv, device)
    v_new = _randn((T, KVH, D), dt, gv, device)
    pad = (slot_t < 0).to(device)
    if bool(pad.any()):
        k_new[pad] = SENTINEL
        v_new[pad] = SENTINEL
    if poison:
        mask = torch.ones(NB * bs, dtype=torch.bool)
        mask[live_t] = False
        # The newest-token slots are overwritten by the write, never poisoned
        # away from it: they are live, so they are already excluded above.
        mask_d = mask.to(device)
        k_cache.view(NB * bs, KVH, D)[mask_d] = float("nan")
        v_cache.view(NB * bs, KVH, D)[mask_d] = float("nan")

    return Workload(
        cfg=cfg, k_cache=k_cache, v_cache=v_cache, q=q, k_new=k_new, v_new=v_new,
        slot_mapping=slot_t.to(device), block_tables=table.to(torch.int32).to(device),
        context_lens=torch.tensor(lens, dtype=torch.int32).to(device),
        scale=1.0 / math.sqrt(D), live_slots=live_t,
        unused_blocks=torch.tensor(unused, dtype=torch.int64))


def make_custom(*, num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, dtype: str = "f32", lens: Sequence[int],
                tail: str = "fill", pad_tokens: int = 0, seed: int = 0,
                num_blocks: Optional[int] = None, device="cpu", poison: bool = False,
                shuffle_write: bool = True) -> Workload:
    """A workload with explicit shape and lengths (tests, random shapes)."""
    cfg = Config(
        name="custom", dtype=dtype, num_seqs=num_seqs, num_heads=num_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        ctx=("explicit", tuple(int(x) for x in lens)), num_blocks=num_blocks,
        tail=tail, pad_tokens=pad_tokens, shuffle_write=shuffle_write, seed=seed)
    return make_workload(cfg, device, poison=poison)


def to_vllm_layout(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """The same stored values in vLLM's cache layout (K [NB, KVH, D/x, bs, x]
    with x elements = 16 bytes, V [NB, KVH, D, bs]): a copy, values unchanged."""
    NB, bs, KVH, D = k_cache.shape
    x = 16 // k_cache.element_size()
    k = k_cache.view(NB, bs, KVH, D // x, x).permute(0, 2, 3, 1, 4).contiguous()
    v = v_cache.permute(0, 2, 3, 1).contiguous()
    return k, v
