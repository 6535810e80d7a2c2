"""Pins of the block-manager oracle (``oracle/block_manager.py``): the
published FNV-1a test vectors, a scenario traced by hand, the prefix-sharing
property of "PagedAttention kernel：paged KV cache 与 block table" (面试官追问:
sequences that share a prompt prefix point at the same physical blocks for it),
and invariants over random operation streams checked by brute force.

Each pin takes the module ``M`` (the real one or a planted-mistake copy).
"""
from __future__ import annotations

import random


def pin_fnv_test_vectors(M):
    """FNV-1a 64-bit, published test vectors."""
    assert M.fnv1a64(b"") == 0xCBF29CE484222325
    assert M.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert M.fnv1a64(b"foobar") == 0x85944171F73967E8
    # the chained key is FNV-1a over the little-endian words (parent, tokens...)
    words = [(1 << 64) - 1, 1, 2]
    assert M.block_hash((1 << 64) - 1, [1, 2]) == M.fnv1a64(b"".join(w.to_bytes(8, "little") for w in words))
    assert M.block_hash(5, [-1]) == M.fnv1a64((5).to_bytes(8, "little") + ((1 << 64) - 1).to_bytes(8, "little"))


def pin_hand_traced_scenario(M):
    """Six blocks of two tokens, traced by hand: sharing of full prefix
    blocks only, a failed allocation that changes nothing, a block registered
    when an append fills it, revival of freed cached blocks, and new blocks
    taken from the front of the free queue."""
    bm = M.BlockManager(6, 2)
    a, ca = bm.add_sequence([1, 2, 3, 4, 5])
    assert (bm.block_table(a), ca, bm.num_free()) == ([0, 1, 2], 0, 3)
    b, cb = bm.add_sequence([1, 2, 3, 4, 9, 9, 7])
    assert (bm.block_table(b), cb, bm.num_free()) == ([0, 1, 3, 4], 4, 1)
    c, cc = bm.add_sequence([1, 2, 8])
    assert (bm.block_table(c), cc, bm.num_free()) == ([0, 5], 2, 0)
    try:
        bm.add_sequence([7])
        raise AssertionError("allocation beyond the pool must fail")
    except M.BlockManagerError:
        pass
    assert bm.num_free() == 0 and bm.block_table(c) == [0, 5]
    bm.free_sequence(a)                                   # block 2 (A's partial block) is freed
    assert bm.num_free() == 1
    assert bm.append(c, 6) == 11                          # position 3 -> block 5, offset 1; [8, 6] fills it
    bm.free_sequence(b)                                   # blocks 1, 3, 4 reach 0 (0 stays with C)
    assert bm.num_free() == 4
    e, ce = bm.add_sequence([1, 2, 3, 4, 9, 9, 5, 5])
    # [1,2] -> 0 (in use), [3,4] -> 1 and [9,9] -> 3 revived, [5,5] new from the queue front (2)
    assert (bm.block_table(e), ce, bm.num_free()) == ([0, 1, 3, 2], 6, 1)
    f, cf = bm.add_sequence([1, 2, 8, 6])                # both blocks cached: C's filled block 5 is shared
    assert (bm.block_table(f), cf) == ([0, 5], 4)
    assert bm.slots(e, 5, 3) == [3 * 2 + 1, 2 * 2 + 0, 2 * 2 + 1]


def pin_eviction_oldest_freed_first(M):
    """When the queue holds only cached blocks, the one freed first is
    reused first, and its prefix is no longer found."""
    bm = M.BlockManager(3, 2)
    s1, _ = bm.add_sequence([1, 1])
    s2, _ = bm.add_sequence([2, 2])
    s3, _ = bm.add_sequence([3, 3])
    bm.free_sequence(s2)
    bm.free_sequence(s1)
    bm.free_sequence(s3)                                 # queue: 1 (s2), 0 (s1), 2 (s3)
    t, c = bm.add_sequence([4, 4])
    assert bm.block_table(t) == [1] and c == 0           # s2's block evicted
    u, c = bm.add_sequence([2, 2])
    assert bm.block_table(u) == [0] and c == 0           # [2,2] is gone; the next oldest (s1's) is taken
    v, c = bm.add_sequence([3, 3])
    assert bm.block_table(v) == [2] and c == 2           # s3's block is still cached: revived


def pin_failure_counts_revived_blocks(M):
    """A sequence that revives the only free (cached) block and needs one new
    block fails, changing nothing: revived blocks are not available for new
    ones."""
    bm = M.BlockManager(2, 2)
    s1, _ = bm.add_sequence([1, 2])
    bm.add_sequence([5])
    bm.free_sequence(s1)                                  # queue: [0], cached [1, 2]
    try:
        bm.add_sequence([1, 2, 3])
        raise AssertionError("needs block 0 revived plus one new block: must fail")
    except M.BlockManagerError:
        pass
    assert list(bm.free) == [0] and bm.refs == [0, 1]
    t, c = bm.add_sequence([1, 2])                         # revival alone fits
    assert bm.block_table(t) == [0] and c == 2


def pin_matching_stops_at_first_miss(M):
    """The first block's entry was evicted while the second's is still
    cached: a new sequence with both reuses neither (cached tokens are a
    contiguous prefix), and the cached second block is evicted in turn."""
    bm = M.BlockManager(4, 2)
    s1, _ = bm.add_sequence([1, 2, 3, 4, 5])              # blocks 0 [1,2], 1 [3,4], 2 [5]
    bm.free_sequence(s1)                                  # queue: 3, 0, 1, 2
    bm.add_sequence([9, 9, 8])                            # takes 3, then 0 (evicting [1,2]); queue: 1, 2
    t, c = bm.add_sequence([1, 2, 3, 4])
    assert c == 0 and bm.block_table(t) == [1, 2]


def pin_collision_guard(M):
    """A block found under the right key but holding other tokens (as after
    a hash collision) is not reused."""
    bm = M.BlockManager(4, 2)
    s1, _ = bm.add_sequence([1, 2])
    b = bm.block_table(s1)[0]
    bm.tokens[b] = [1, 3]                                 # forge the colliding entry
    t, c = bm.add_sequence([1, 2])
    assert c == 0 and bm.block_table(t) != [b]


def pin_prefix_sharing_property(M):
    """Two sequences whose first k*bs tokens agree share exactly their first
    k blocks (the partial block and everything after the first difference
    are private)."""
    rng = random.Random(7)
    for bs in (1, 2, 4, 16):
        for _ in range(20):
            k = rng.randrange(0, 5)
            prefix = [rng.randrange(50) for _ in range(k * bs)]
            x = prefix + [100 + rng.randrange(50) for _ in range(rng.randrange(1, 3 * bs))]
            y = prefix + [200 + rng.randrange(50) for _ in range(rng.randrange(1, 3 * bs))]
            bm = M.BlockManager(64, bs)
            sx, cx = bm.add_sequence(x)
            sy, cy = bm.add_sequence(y)
            tx, ty = bm.block_table(sx), bm.block_table(sy)
            assert cx == 0 and cy == k * bs
            assert tx[:k] == ty[:k] and not (set(tx[k:]) & set(ty[k:])) and not (set(tx[k:]) & set(ty[:k]))


def _check_invariants(M, bm, model):
    nb = bm.nb
    refs = [0] * nb
    for sid, toks in model.items():
        table = bm.block_table(sid)
        assert len(table) == -(-len(toks) // bm.bs) and bm.length(sid) == len(toks)
        for b in table:
            refs[b] += 1
        # every position's slot is in its block
        for p, s in enumerate(bm.slots(sid, 0, len(toks))):
            assert s // bm.bs == table[p // bm.bs] and s % bm.bs == p % bm.bs
        # full blocks shared between sequences hold the same tokens
    assert refs == bm.refs
    free = list(bm.free)
    assert len(set(free)) == len(free) and all(refs[b] == 0 for b in free)
    assert sorted(free + [b for b in range(nb) if refs[b] > 0]) == list(range(nb))
    for key, b in bm.by_hash.items():
        assert bm.hash[b] == key and len(bm.tokens[b]) == bm.bs
    # a block in two tables is a full block whose tokens both sequences hold at that index
    owners = {}
    for sid, toks in model.items():
        for i, b in enumerate(bm.block_table(sid)):
            chunk = toks[i * bm.bs:(i + 1) * bm.bs]
            if b in owners:
                assert len(chunk) == bm.bs and owners[b] == chunk
            owners[b] = chunk


def pin_random_streams_invariants(M):
    """Random add / append / free streams over prompts drawn from a few shared
    prefixes: reference counts equal table occupancy, the queue holds exactly
    the unreferenced blocks, slots follow the tables, shared blocks hold equal
    tokens, and failures change nothing."""
    rng = random.Random(11)
    for trial in range(30):
        bs = rng.choice([1, 2, 3, 4, 8])
        bm = M.BlockManager(rng.randrange(4, 40), bs)
        prefixes = [[rng.randrange(20) for _ in range(rng.randrange(0, 4 * bs))] for _ in range(3)]
        model = {}
        for step in range(60):
            op = rng.random()
            if op < 0.45 or not model:
                toks = rng.choice(prefixes) + [rng.randrange(20) for _ in range(rng.randrange(0, 2 * bs))]
                before = (list(bm.free), dict(bm.by_hash), list(bm.refs))
                try:
                    sid, cached = bm.add_sequence(toks)
                    model[sid] = list(toks)
                    assert cached % bs == 0 and cached <= len(toks)
                except M.BlockManagerError:
                    assert (list(bm.free), dict(bm.by_hash), list(bm.refs)) == before
            elif op < 0.8:
                sid = rng.choice(sorted(model))
                t = rng.randrange(20)
                try:
                    slot = bm.append(sid, t)
                    model[sid].append(t)
                    assert slot == bm.slots(sid, len(model[sid]) - 1, 1)[0]
                except M.BlockManagerError:
                    assert bm.num_free() == 0
            else:
                sid = rng.choice(sorted(model))
                bm.free_sequence(sid)
                del model[sid]
            _check_invariants(M, bm, model)


ALL_PINS = [
    pin_fnv_test_vectors,
    pin_hand_traced_scenario,
    pin_eviction_oldest_freed_first,
    pin_failure_counts_revived_blocks,
    pin_matching_stops_at_first_miss,
    pin_collision_guard,
    pin_prefix_sharing_property,
    pin_random_streams_invariants,
]
