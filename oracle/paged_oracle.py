"""CPU oracle for the paged KV-cache write and paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers or constants) and imports nothing from it.

It is a plain, slow, obviously correct restatement of what the pages define,
in NumPy float64 over the exact stored values (fp32, or bf16 given as raw
uint16 bit patterns and widened exactly).

Sources (titles of the pages, with the section each function follows):
  [P1] "P09 · Paged KV 写入 + decode attention（参考实现）", kuanzhou.online
       sections 题面速览 (problem statement), 框架视角 · shape trace (the two step
       tables), 不变量 (invariants I1-I5), 细节 and L2 思路.
  [P2] "PagedAttention kernel：paged KV cache 与 block table",
       inference-learning-path.pages.dev, sections 直接答案 and 代码 (the
       online-softmax fold over the block table).

The vLLM cache layout of [P2] 深入原理 (K as [NB, KVH, D/x, bs, x], V as
[NB, KVH, D, bs]) is handled by plain re-indexing into [P1]'s layout and back
(``pack_*`` / ``unpack_*``): it moves stored values, never changes them.

``prefill`` (several new queries per sequence) is the varlen version [P1]
asks for in 面试官追问 & 对照源码 without defining it; it takes the plainest
reading that [P1] 细节 supports (see its docstring).

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
the pages print, closed forms, invariants and brute force; none is "parity
unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "stored_to_f64",
    "slot_to_block_offset",
    "blocks_needed",
    "kv_head_of",
    "write_kv",
    "gather_context",
    "decode",
    "decode_online_fold",
    "query_positions",
    "prefill",
    "vllm_pack_width",
    "pack_k_vllm",
    "pack_v_vllm",
    "unpack_k_vllm",
    "unpack_v_vllm",
    "write_kv_vllm",
    "decode_vllm",
    "OracleError",
]


class OracleError(ValueError):
    """An input violates a precondition the pages state or imply."""


# ---------------------------------------------------------------------------
# Stored values -> float64
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns.

    A bfloat16 is the upper 16 bits of an IEEE binary32; shifting the pattern
    into the high half of a 32-bit word gives that binary32 exactly, and
    binary32 -> binary64 is exact.
    """
    b = np.asarray(bits)
    if b.dtype not in (np.uint16, np.int16):
        raise OracleError("bf16 values must be passed as 16-bit patterns")
    w = (b.astype(np.uint16).astype(np.uint32) << np.uint32(16))
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns stay NaN
        return w.view(np.float32).astype(np.float64)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored cache/query values to float64 without rounding ([P1] 细节:
    q, k and v may all be taken to fp32 for scores, softmax and the weighted
    sum; fp64 is a superset)."""
    if dtype == "f32":
        a = np.asarray(a)
        if a.dtype != np.float32:
            raise OracleError("f32 values must be float32")
        return a.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise OracleError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Index arithmetic ([P1] 直觉与类比 and 细节: slot = block * bs + offset, so
# cache[slot // bs, slot % bs] is the slot-th row of the flattened cache)
# ---------------------------------------------------------------------------

def slot_to_block_offset(slot: int, block_size: int) -> tuple[int, int]:
    if slot < 0:
        raise OracleError("negative slots are padding and have no position")
    return slot // block_size, slot % block_size


def blocks_needed(n: int, block_size: int) -> int:
    """Table entries sequence of length n uses: ceil(n / bs), not n // bs
    ([P1] shape trace, decode step 1)."""
    return -(-int(n) // int(block_size))


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """GQA: query head h reads kv head h // (H / KVH) — the repeat_interleave
    mapping ([P1] 题面速览; shape trace, decode step 5; invariant I5)."""
    if num_heads % num_kv_heads:
        raise OracleError("num_heads must be a multiple of num_kv_heads")
    return h // (num_heads // num_kv_heads)


# ---------------------------------------------------------------------------
# write_kv ([P1] 题面速览 "写", shape trace write_kv steps 1-4, L2 思路)
# ---------------------------------------------------------------------------

def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k: np.ndarray,
             v: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Scatter token i's K/V rows into cache[slot // bs, slot % bs], in place.

    Negative slots are padding and are skipped (the statement names -1; its
    code keeps ``slot >= 0``, so every negative value is skipped).  Stored bits
    are copied unchanged.  Valid slots must be in range and distinct (the pages
    are silent on duplicates; this is taken as a precondition).
    Returns None: the caller's arrays are the result.
    """
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    if v_cache.shape != k_cache.shape:
        raise OracleError("k_cache and v_cache shapes differ")
    T = len(slot_mapping)
    if k.shape[0] != T or v.shape[0] != T:
        raise OracleError("k/v rows must match slot_mapping length")
    if k.shape[1:] != k_cache.shape[2:] or v.shape[1:] != v_cache.shape[2:]:
        raise OracleError("k/v rows must be [KVH, D] like the cache")
    seen = set()
    for i in range(T):
        s = int(slot_mapping[i])
        if s < 0:
            continue
        if s >= NB * bs:
            raise OracleError(f"slot {s} beyond the cache ({NB} blocks of {bs})")
        if s in seen:
            raise OracleError(f"slot {s} written twice")
        seen.add(s)
        blk, off = slot_to_block_offset(s, bs)
        k_cache[blk, off] = k[i]
        v_cache[blk, off] = v[i]
    return None


# ---------------------------------------------------------------------------
# decode ([P1] 题面速览 "decode 读", shape trace decode steps 1-7)
# ---------------------------------------------------------------------------

def gather_context(cache: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """K (or V) rows of a sequence of length n, in logical order.

    Only the first ceil(n / bs) table entries are read (invariant I2); the
    gathered blocks are taken in table order (no sorting), flattened to a
    token axis and cut to exactly n rows (invariant I3).
    Returns [n, KVH, D] in the cache's stored dtype.
    """
    NB, bs = cache.shape[0], cache.shape[1]
    nb = blocks_needed(n, bs)
    if nb > len(table_row):
        raise OracleError(f"context of {n} tokens needs {nb} table entries, table has {len(table_row)}")
    tbl = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and (tbl.min() < 0 or tbl.max() >= NB):
        raise OracleError("table entry outside the block pool")
    blocks = cache[tbl]                                   # [nb, bs, KVH, D]
    flat = blocks.reshape(nb * bs, *cache.shape[2:])      # token axis
    return flat[:n]


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
           dtype: str) -> np.ndarray:
    """Paged decode attention for one query per sequence, in float64.

    out[b, h] = softmax_j(scale * q[b, h] . K_b[j, kvh]) . V_b[:, kvh]
    with K_b, V_b the first n_b gathered rows and kvh = h // (H / KVH).  The
    scale multiplies the scores before the softmax.  Paging does not change
    the result (exactly dense attention, [P2] 直接答案), so this is the plain
    definition, computed directly (max-shifted exponentials, then normalised).
    n_b = 0 gives zeros (a reading: the pages imply n >= 1 in decode).
    Returns the unrounded float64 result [B, H, D].
    """
    B, H, D = q.shape
    KVH = k_cache.shape[2]
    if k_cache.shape[3] != D:
        raise OracleError("head_dim of q and cache differ")
    if H % KVH:
        raise OracleError("num_heads must be a multiple of num_kv_heads")
    qf = stored_to_f64(q, dtype)
    out = np.zeros((B, H, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        if n < 0:
            raise OracleError("negative context length")
        if n == 0:
            continue
        Kb = stored_to_f64(gather_context(k_cache, block_tables[b], n), dtype)  # [n, KVH, D]
        Vb = stored_to_f64(gather_context(v_cache, block_tables[b], n), dtype)
        for h in range(H):
            kvh = kv_head_of(h, H, KVH)
            s = scale * (Kb[:, kvh, :] @ qf[b, h])        # [n] scores, scaled first
            e = np.exp(s - s.max())
            p = e / e.sum()
            out[b, h] = p @ Vb[:, kvh, :]
    return out


def decode_online_fold(q, k_cache, v_cache, block_tables, context_lens, scale,
                       dtype: str) -> np.ndarray:
    """Second, independent formulation: walk each table entry by entry and fold
    one token at a time into a running (max, sum, accumulator), as [P2] 代码
    describes: m' = max(m, s); c = exp(m - m') (0 while m is -inf);
    l' = l c + exp(s - m'); acc' = acc c + exp(s - m') v; result acc / l.

    Pure Python scalar loops — only for tiny shapes.
    """
    B, H, D = q.shape
    NB, bs, KVH, _ = k_cache.shape
    qf = stored_to_f64(q, dtype)
    kf = stored_to_f64(k_cache, dtype)
    vf = stored_to_f64(v_cache, dtype)
    out = np.zeros((B, H, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        for h in range(H):
            kvh = kv_head_of(h, H, KVH)
            m, l = -math.inf, 0.0
            acc = [0.0] * D
            pos = 0
            for j in range(blocks_needed(n, bs)):
                phys = int(block_tables[b][j])
                for t in range(bs):
                    if pos >= n:
                        break
                    s = scale * sum(float(qf[b, h, d]) * float(kf[phys, t, kvh, d]) for d in range(D))
                    m_new = max(m, s)
                    c = math.exp(m - m_new) if m != -math.inf else 0.0
                    p = math.exp(s - m_new)
                    l = l * c + p
                    acc = [acc[d] * c + p * float(vf[phys, t, kvh, d]) for d in range(D)]
                    m = m_new
                    pos += 1
            if n:
                out[b, h] = [a / l for a in acc]
    return out


# ---------------------------------------------------------------------------
# prefill: many new queries per sequence ([P1] 面试官追问 asks for the varlen
# prefill version; [P1] 细节 gives the reason decode has no causal mask)
# ---------------------------------------------------------------------------

def query_positions(n: int, num_queries: int) -> np.ndarray:
    """Positions of a sequence's new queries: they are its last num_queries
    tokens (already written into the cache, as the newest token is in decode,
    [P1] 细节), so query i sits at position n - num_queries + i."""
    if num_queries < 0 or num_queries > n:
        raise OracleError(f"{num_queries} new queries do not fit a context of {n} tokens")
    return np.arange(n - num_queries, n, dtype=np.int64)


def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray,
            query_start_loc: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Paged attention of a packed (varlen) batch of new queries, in float64.

    Reading of the pages (they pose the question and stop there):
      * q is [T, H, D]: sequence b owns rows query_start_loc[b] ..
        query_start_loc[b+1] - 1 (query_start_loc[0] = 0, non-decreasing,
        query_start_loc[B] = T), L_b of them;
      * context_lens[b] = n_b counts every token of the sequence, the L_b new
        ones included (their K/V rows are written before the call, as decode's
        newest token is), and query i of the sequence is token n_b - L_b + i;
      * decode needs no causal mask only because its one query is the newest
        token ([P1] 细节); with several, query at position p attends to the
        tokens 0..p of the gathered context and to nothing after it;
      * everything else is decode's definition: the same gather (table order,
        ceil(n/bs) entries, cut to n rows), the GQA map h // (H/KVH), the scale
        on the scores before the softmax.
    L_b = 1 for every b is exactly decode.  Returns the unrounded float64
    output [T, H, D]; rows of no sequence (none, given the preconditions) stay 0.
    """
    T, H, D = q.shape
    KVH = k_cache.shape[2]
    if k_cache.shape[3] != D:
        raise OracleError("head_dim of q and cache differ")
    if H % KVH:
        raise OracleError("num_heads must be a multiple of num_kv_heads")
    qs = np.asarray(query_start_loc, dtype=np.int64)
    B = len(context_lens)
    if len(qs) != B + 1 or qs[0] != 0 or qs[-1] != T or np.any(np.diff(qs) < 0):
        raise OracleError("query_start_loc must run from 0 to T without decreasing")
    qf = stored_to_f64(q, dtype)
    out = np.zeros((T, H, D), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        s0, s1 = int(qs[b]), int(qs[b + 1])
        pos = query_positions(n, s1 - s0)
        if s1 == s0:
            continue
        Kb = stored_to_f64(gather_context(k_cache, block_tables[b], n), dtype)   # [n, KVH, D]
        Vb = stored_to_f64(gather_context(v_cache, block_tables[b], n), dtype)
        visible = np.arange(n)[None, :] <= pos[:, None]                          # [L, n] causal mask
        for h in range(H):
            kvh = kv_head_of(h, H, KVH)
            s = scale * (qf[s0:s1, h, :] @ Kb[:, kvh, :].T)                     # [L, n], scaled first
            s = np.where(visible, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            out[s0:s1, h] = p @ Vb[:, kvh, :]
    return out


# ---------------------------------------------------------------------------
# vLLM's cache layout ([P2] 深入原理: the K cache's extra dimension)
# ---------------------------------------------------------------------------

def vllm_pack_width(dtype: str) -> int:
    """x = 16 bytes / element size: the innermost K dimension packs one
    16-byte-aligned group of head_dim ([P2] 深入原理: 8 for 2-byte types)."""
    return {"bf16": 8, "f32": 4}[dtype]


def pack_k_vllm(k_cache: np.ndarray, dtype: str) -> np.ndarray:
    """[NB, bs, KVH, D] -> [NB, KVH, D/x, bs, x]: element (blk, t, h, d) moves
    to (blk, h, d // x, t, d % x)."""
    NB, bs, KVH, D = k_cache.shape
    x = vllm_pack_width(dtype)
    if D % x:
        raise OracleError("head_dim must be a multiple of the pack width")
    return np.ascontiguousarray(k_cache.reshape(NB, bs, KVH, D // x, x).transpose(0, 2, 3, 1, 4))


def unpack_k_vllm(k_packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_k_vllm: [NB, KVH, D/x, bs, x] -> [NB, bs, KVH, D]."""
    NB, KVH, G, bs, x = k_packed.shape
    return np.ascontiguousarray(k_packed.transpose(0, 3, 1, 2, 4).reshape(NB, bs, KVH, G * x))


def pack_v_vllm(v_cache: np.ndarray) -> np.ndarray:
    """[NB, bs, KVH, D] -> [NB, KVH, D, bs]: V is read along the token axis and
    needs no packing ([P2] 深入原理)."""
    return np.ascontiguousarray(v_cache.transpose(0, 2, 3, 1))


def unpack_v_vllm(v_packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_v_vllm: [NB, KVH, D, bs] -> [NB, bs, KVH, D]."""
    return np.ascontiguousarray(v_packed.transpose(0, 3, 1, 2))


def write_kv_vllm(k_packed: np.ndarray, v_packed: np.ndarray, k: np.ndarray, v: np.ndarray,
                  slot_mapping: np.ndarray) -> None:
    """write_kv on caches in vLLM's layout, in place: the same scatter, done in
    [P1]'s layout and re-indexed back (the layout moves values only)."""
    x = k_packed.shape[4]
    dtype = "bf16" if x == 8 else "f32"
    kc, vc = unpack_k_vllm(k_packed), unpack_v_vllm(v_packed)
    write_kv(kc, vc, k, v, slot_mapping)
    k_packed[...] = pack_k_vllm(kc, dtype)
    v_packed[...] = pack_v_vllm(vc)
    return None


def decode_vllm(q, k_packed, v_packed, block_tables, context_lens, scale, dtype: str) -> np.ndarray:
    """decode on caches in vLLM's layout: paging and layout change where the
    rows live, not what attention computes ([P2] 直接答案)."""
    return decode(q, unpack_k_vllm(k_packed), unpack_v_vllm(v_packed), block_tables, context_lens,
                  scale, dtype)
