"""The block-manager oracle against its pins, and planted mistakes (each must
fail at least one pin).  CPU only."""
import os
import types

import pytest

import oracle.block_manager as M
from tests.block_manager_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block_manager.py")

MUTANTS = {
    "fnv_prime_wrong": ("FNV_PRIME = 0x100000001B3", "FNV_PRIME = 0x100000001B5"),
    "fnv_multiply_then_xor": ("        h ^= byte\n        h = (h * FNV_PRIME) & _MASK",
                              "        h = (h * FNV_PRIME) & _MASK\n        h ^= byte"),
    "hash_ignores_parent": ("    words = [parent & _MASK] + [int(t) & _MASK for t in tokens]",
                            "    words = [int(t) & _MASK for t in tokens]"),
    "no_token_check": ("        if b is not None and self.tokens[b] == list(toks):", "        if b is not None:"),
    "lifo_free_queue": ("        b = self.free.popleft()", "        b = self.free.pop()"),
    "eviction_keeps_hash": ("            del self.by_hash[self.hash[b]]\n", "            pass\n"),
    "match_after_miss": ("            if len(reused) == i:\n", "            if True:\n"),
    "share_partial_block": ("        nfull, nblocks = n // bs, -(-n // bs)", "        nfull, nblocks = -(-n // bs), -(-n // bs)"),
    "freed_block_to_front": ("                self.free.append(b)", "                self.free.appendleft(b)"),
    "no_refcount_on_reuse": ("            self.refs[b] += 1\n", "            self.refs[b] = 1\n"),
    "full_block_not_registered_on_append": ("            self._register(b, key, tokens[i * self.bs:(i + 1) * self.bs])\n", "            pass\n"),
    "failure_check_ignores_revival": ("        if len(self.free) - len(revive) < nblocks - len(reused):",
                                      "        if len(self.free) < nblocks - len(reused):"),
}


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(M)


def _mutant(name):
    src = open(SRC, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mod = types.ModuleType(f"bm_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    Mm = _mutant(name)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(Mm)
        except Exception as e:  # noqa: BLE001 - any failure counts
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin catches mutant {name}"
