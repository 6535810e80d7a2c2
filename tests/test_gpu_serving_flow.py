"""A serving flow driven by the C++ block manager on an MI355X, held to the
oracle end to end.

Five requests share a 48-token system prompt (three full blocks of 16).  The
manager shares the prompt's blocks, reports the cached prefix, and gives the
slots of the uncached tokens; pa_write_kv writes them and pa_prefill attends
(chunked prefill over the cached prefix).  Three decode steps follow:
append -> slot -> pa_write_kv -> pa_decode over tables the manager fills.
Each decode step also runs pa_decode_shared_prefix with the cached prompt
length the manager reported as the hint.  Then one request is freed and
re-added: its prefix blocks are revived and only its tail is prefilled again.

The oracle side runs the same flow with the oracle's block manager, write,
prefill and decode.  K/V rows are a fixed function of (token id, position),
as a model's would be, so shared prefixes hold identical values.  Tables and
slots must agree exactly; attention outputs within the bf16 tolerance.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import oracle.block_manager as OBM
import paged_kv_cache_70_amd as pk
from tests.gpu_util import assert_matches_oracle, stored_np

pytestmark = pytest.mark.gpu

NB, BS, KVH, H, D, VOCAB, MAXPOS = 256, 16, 2, 8, 128, 40, 320


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[gpu-serving] {msg}", flush=True)
    sys.stdout.flush()


class Flow:
    """The same flow on the GPU (C++ manager, HIP kernels) and on the oracle."""

    def __init__(self):
        g = torch.Generator().manual_seed(61)
        rnd = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
        self.kv_k = rnd(VOCAB, MAXPOS, KVH, D)          # K row of token t at position p
        self.kv_v = rnd(VOCAB, MAXPOS, KVH, D)
        self.qtab = rnd(VOCAB, MAXPOS, H, D)            # q row of token t at position p
        self.kc = torch.zeros((NB, BS, KVH, D), dtype=torch.bfloat16, device="cuda")
        self.vc = torch.zeros_like(self.kc)
        self.ko = stored_np(self.kc.cpu()).copy()       # oracle caches (bit patterns)
        self.vo = stored_np(self.vc.cpu()).copy()
        self.bm, self.obm = pk.BlockManager(NB, BS), OBM.BlockManager(NB, BS)
        self.tokens = {}                                # seq id -> token ids
        self.scale = 1.0 / np.sqrt(D)

    def rows(self, tab, toks, positions):
        return tab[torch.tensor(toks), torch.tensor(positions)]

    def write(self, sids, starts):
        """Write positions start.. of each sequence (the uncached / new tokens)."""
        toks, pos, slots = [], [], []
        for sid, st in zip(sids, starts):
            t = self.tokens[sid]
            s_g = self.bm.slots(sid, st, len(t) - st)
            s_o = self.obm.slots(sid, st, len(t) - st)
            assert s_g == s_o, "slots"
            toks += t[st:]
            pos += list(range(st, len(t)))
            slots += s_g
        k, v = self.rows(self.kv_k, toks, pos), self.rows(self.kv_v, toks, pos)
        sl = torch.tensor(slots, dtype=torch.int64)
        pk.write_kv(self.kc, self.vc, k.cuda(), v.cuda(), sl.cuda())
        O.write_kv(self.ko, self.vo, stored_np(k), stored_np(v), sl.numpy())
        return toks, pos

    def tables(self, sids):
        W = max(len(self.obm.block_table(s)) for s in sids) + 1
        tab, lens = self.bm.fill_tables(sids, W, fill=99999)
        for i, s in enumerate(sids):
            row = self.obm.block_table(s)
            assert tab[i, :len(row)].tolist() == row and lens[i] == self.obm.length(s), "tables"
        return tab, lens

    def prefill(self, sids, cached):
        toks, pos = self.write(sids, cached)
        tab, lens = self.tables(sids)
        new = [len(self.tokens[s]) - c for s, c in zip(sids, cached)]
        qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        q = self.rows(self.qtab, toks, pos)
        out = pk.prefill(q.cuda(), self.kc, self.vc, torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(),
                         torch.from_numpy(qsl).cuda(), self.scale)
        torch.cuda.synchronize()
        ref = O.prefill(stored_np(q), self.ko, self.vo, tab, lens, qsl, self.scale, "bf16")
        return out, ref

    def decode(self, sids, shared_tokens=0):
        steps_tok = [int((7 * s + len(self.tokens[s])) % VOCAB) for s in sids]
        for s, t in zip(sids, steps_tok):
            slot_g, slot_o = self.bm.append(s, t), self.obm.append(s, t)
            assert slot_g == slot_o, "append slot"
            self.tokens[s].append(t)
        self.write(sids, [len(self.tokens[s]) - 1 for s in sids])
        tab, lens = self.tables(sids)
        q = self.rows(self.qtab, steps_tok, [len(self.tokens[s]) - 1 for s in sids])
        args = (q.cuda(), self.kc, self.vc, torch.from_numpy(tab).cuda(), torch.from_numpy(lens).cuda(), self.scale)
        out = pk.decode(*args)
        # the same step with the shared prompt as the hint (partitions of one
        # block, so that the 48 shared tokens are 3 whole partitions)
        out_sp = pk.decode_shared_prefix(*args, shared_tokens, partition_size=BS) if shared_tokens else None
        torch.cuda.synchronize()
        ref = O.decode(stored_np(q), self.ko, self.vo, tab, lens, self.scale, "bf16")
        return out, out_sp, ref

    def add(self, toks):
        r_g = self.bm.add_sequence(toks)
        r_o = self.obm.add_sequence(toks)
        assert r_g == r_o, "add_sequence"
        self.tokens[r_g[0]] = list(toks)
        return r_g


def test_serving_flow_with_shared_prompt():
    f = Flow()
    rng = np.random.default_rng(62)
    system = rng.integers(0, VOCAB, 48).tolist()
    prompts = [system + rng.integers(0, VOCAB, n).tolist() for n in (5, 16, 37, 1, 60)]
    added = [f.add(p) for p in prompts]
    sids = [s for s, _ in added]
    cached = [c for _, c in added]
    assert cached == [0, 48, 48, 48, 48]            # the first request writes the prompt; the rest share it
    tables = [f.bm.block_table(s) for s in sids]
    assert all(t[:3] == tables[0][:3] for t in tables)
    out, ref = f.prefill(sids, cached)
    err = assert_matches_oracle(out, ref, "bf16", "prefill over a shared prompt")
    _say(f"prefill: {sum(len(p) - c for p, c in zip(prompts, cached))} new tokens, max err {err:.2e}")
    for step in range(3):
        out, out_sp, ref = f.decode(sids, shared_tokens=cached[1])
        err = assert_matches_oracle(out, ref, "bf16", f"decode step {step}")
        err_sp = assert_matches_oracle(out_sp, ref, "bf16", f"shared-prefix decode step {step}")
        _say(f"decode step {step}: max err {err:.2e} (shared-prefix decode {err_sp:.2e})")
    # free request 2 and bring it back: its full blocks are revived from the cache
    gone = sids[2]
    toks = list(f.tokens[gone])
    f.bm.free_sequence(gone)
    f.obm.free_sequence(gone)
    del f.tokens[gone]
    sid, c = f.add(toks)
    assert c == (len(toks) // BS) * BS
    out, ref = f.prefill([sid], [c])
    err = assert_matches_oracle(out, ref, "bf16", "prefill after revival")
    _say(f"re-added request: {c} cached tokens, {len(toks) - c} prefilled, max err {err:.2e}")
