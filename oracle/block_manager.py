"""CPU oracle for the host block manager with prefix sharing.

TEST INFRASTRUCTURE ONLY, like ``oracle.paged_oracle``: only the tests, the
smoke check and the benchmark's CPU baseline use it; it shares no code with the
C++ manager in the library and imports nothing from it.

Sources:
  [P2] "PagedAttention kernel：paged KV cache 与 block table", 直接答案 and
       面试官追问: blocks live anywhere in a shared pool; sequences whose
       prompts share a prefix point their tables at the same physical blocks
       for it (prefix caching), so the prefix is computed and stored once.
  [P3] the third page (a C++ engine's write-up), its BlockManager: a pool of
       fixed-size blocks; each block keeps its token ids and a hash of its
       tokens chained with its prefix's hash; a hash -> block map; a queue of
       free block ids and a set of used ones; allocate(token ids) fills a block
       table and reports how many leading tokens are already cached.

The pages stop there (reference counts are commented out, eviction is a
to-do).  The reading taken, step by step:
  * block i of a sequence holds positions [i*bs, (i+1)*bs);
  * a full block's key is the chained hash h_i = FNV-1a-64 of the 8-byte
    little-endian words (h_{i-1}, t_0, ..., t_{bs-1}), with h_{-1} = -1
    (all ones) as [P3]'s default prefix; a cached block is reused only when
    its stored tokens equal the new ones too (a guard against collisions);
  * adding a sequence walks its full blocks from the start and reuses cached
    blocks until the first block that is not cached; every later block,
    including a partial last one, is new; the result reports
    (reused blocks) * bs cached tokens;
  * a partial block is never shared; a block is registered for sharing when
    it is full (at allocation, or when an appended token fills it), unless
    its hash is already registered;
  * blocks have reference counts; freeing a sequence decrements them; a block
    whose count reaches 0 goes to the back of the free queue and keeps its
    hash and tokens, so a later sequence can revive it (it then leaves the
    queue);
  * new blocks come from the front of the queue (initially 0, 1, ..., NB-1):
    the oldest freed cached block is evicted first, and its hash entry is
    dropped when it is reused;
  * an operation that needs more blocks than the queue holds (after the
    revived ones) fails and changes nothing.
Every function here is pinned by tests/test_block_manager_oracle.py.
"""
from __future__ import annotations

from collections import deque

__all__ = ["FNV_OFFSET", "FNV_PRIME", "fnv1a64", "block_hash", "BlockManagerError", "BlockManager"]

FNV_OFFSET = 0xCBF29CE484222325   # FNV-1a 64-bit offset basis (published)
FNV_PRIME = 0x100000001B3         # FNV 64-bit prime (published)
_MASK = (1 << 64) - 1
NO_PARENT = _MASK                 # h_{-1}: -1 as an unsigned 64-bit word


def fnv1a64(data: bytes) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the prime."""
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & _MASK
    return h


def block_hash(parent: int, tokens) -> int:
    """Chained key of a full block: FNV-1a-64 over the little-endian 8-byte
    words (parent, t_0, ..., t_{bs-1}), token ids as signed 64-bit."""
    words = [parent & _MASK] + [int(t) & _MASK for t in tokens]
    return fnv1a64(b"".join(w.to_bytes(8, "little") for w in words))


class BlockManagerError(RuntimeError):
    """Not enough free blocks, or an unknown sequence; nothing was changed."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.nb, self.bs = num_blocks, block_size
        self.refs = [0] * num_blocks
        self.hash = [None] * num_blocks          # key of a registered full block
        self.tokens = [None] * num_blocks        # its token ids
        self.free = deque(range(num_blocks))     # front: next to hand out
        self.by_hash = {}                        # key -> block id
        self.seqs = {}                           # seq id -> (tokens, block ids, hashes of full blocks)
        self.next_seq = 0

    # -- helpers -----------------------------------------------------------
    def _take(self) -> int:
        """A new block from the front of the queue; a cached block there is
        evicted (its key dropped)."""
        b = self.free.popleft()
        if self.hash[b] is not None:
            del self.by_hash[self.hash[b]]
            self.hash[b] = None
            self.tokens[b] = None
        self.refs[b] = 1
        return b

    def _register(self, b: int, key: int, toks) -> None:
        if key not in self.by_hash:
            self.by_hash[key] = b
            self.hash[b] = key
            self.tokens[b] = list(toks)

    def _lookup(self, key: int, toks):
        b = self.by_hash.get(key)
        if b is not None and self.tokens[b] == list(toks):
            return b
        return None

    # -- operations ----------------------------------------------------------
    def add_sequence(self, tokens) -> tuple[int, int]:
        """New sequence holding `tokens`; returns (seq id, cached tokens)."""
        tokens = [int(t) for t in tokens]
        bs, n = self.bs, len(tokens)
        nfull, nblocks = n // bs, -(-n // bs)
        # plan: leading cached blocks, then new ones
        reused, keys, parent = [], [], NO_PARENT
        for i in range(nfull):
            key = block_hash(parent, tokens[i * bs:(i + 1) * bs])
            keys.append(key)
            parent = key
            if len(reused) == i:
                b = self._lookup(key, tokens[i * bs:(i + 1) * bs])
                if b is not None:
                    reused.append(b)
        revive = [b for b in reused if self.refs[b] == 0]
        if len(self.free) - len(revive) < nblocks - len(reused):
            raise BlockManagerError("not enough free blocks")
        for b in reused:
            if self.refs[b] == 0:
                self.free.remove(b)
            self.refs[b] += 1
        blocks = list(reused)
        for i in range(len(reused), nblocks):
            b = self._take()
            if i < nfull:
                self._register(b, keys[i], tokens[i * bs:(i + 1) * bs])
            blocks.append(b)
        sid = self.next_seq
        self.next_seq += 1
        self.seqs[sid] = (tokens, blocks, keys)
        return sid, len(reused) * bs

    def append(self, sid: int, token: int) -> int:
        """Append one token; returns its slot (block * bs + offset)."""
        if sid not in self.seqs:
            raise BlockManagerError("unknown sequence")
        tokens, blocks, keys = self.seqs[sid]
        pos = len(tokens)
        if pos % self.bs == 0:
            if not self.free:
                raise BlockManagerError("not enough free blocks")
            blocks.append(self._take())
        tokens.append(int(token))
        b = blocks[pos // self.bs]
        if pos % self.bs == self.bs - 1:                    # the block just filled up
            i = pos // self.bs
            key = block_hash(keys[i - 1] if i else NO_PARENT, tokens[i * self.bs:(i + 1) * self.bs])
            keys.append(key)
            self._register(b, key, tokens[i * self.bs:(i + 1) * self.bs])
        return b * self.bs + pos % self.bs

    def free_sequence(self, sid: int) -> None:
        if sid not in self.seqs:
            raise BlockManagerError("unknown sequence")
        _, blocks, _ = self.seqs.pop(sid)
        for b in blocks:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)

    def block_table(self, sid: int) -> list:
        return list(self.seqs[sid][1])

    def length(self, sid: int) -> int:
        return len(self.seqs[sid][0])

    def slots(self, sid: int, start: int, count: int) -> list:
        """Slots of positions start .. start + count - 1 of the sequence."""
        tokens, blocks, _ = self.seqs[sid]
        if start < 0 or count < 0 or start + count > len(tokens):
            raise BlockManagerError("positions outside the sequence")
        return [blocks[p // self.bs] * self.bs + p % self.bs for p in range(start, start + count)]

    def num_free(self) -> int:
        return len(self.free)
