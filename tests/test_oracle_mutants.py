"""Negative controls: each plausible mistake, planted in a copy of the oracle
on the CPU, must fail at least one pin.  The mistakes include the bug table of
"P09 · Paged KV 写入 + decode attention（参考实现）" (section 易错点: no -1
filter, reading the whole table row, no truncation, repeat instead of
repeat_interleave) and generic slips (a dropped term, a wrong index, a
transposed operand, a swapped K/V).
"""
import os
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paged_oracle.py")

MUTANTS = {
    # write side
    "no_negative_filter": ("        if s < 0:\n            continue\n        if s >= NB * bs:",
                           "        if s >= NB * bs:"),
    "minus_one_wraps_to_last_slot": (
        "        if s < 0:\n            continue\n        if s >= NB * bs:",
        "        s = s % (NB * bs)\n        if s >= NB * bs:"),
    "write_swaps_kv": ("        k_cache[blk, off] = k[i]\n        v_cache[blk, off] = v[i]",
                       "        k_cache[blk, off] = v[i]\n        v_cache[blk, off] = k[i]"),
    "offset_block_swapped": ("    return slot // block_size, slot % block_size",
                             "    return slot % block_size, slot // block_size"),
    # decode side
    "floor_block_count": ("    return -(-int(n) // int(block_size))",
                          "    return max(1, int(n) // int(block_size))"),
    "whole_table_row": ("    nb = blocks_needed(n, bs)\n    if nb > len(table_row):",
                        "    nb = len(table_row)\n    if nb > len(table_row):"),
    "no_truncation": ("    return flat[:n]", "    return flat[:nb * bs]"),
    "sorted_table": ("    tbl = np.asarray(table_row[:nb], dtype=np.int64)",
                     "    tbl = np.sort(np.asarray(table_row[:nb], dtype=np.int64))"),
    "gqa_repeat": ("    return h // (num_heads // num_kv_heads)", "    return h % num_kv_heads"),
    "scale_dropped": ("            s = scale * (Kb[:, kvh, :] @ qf[b, h])",
                      "            s = (Kb[:, kvh, :] @ qf[b, h])"),
    "scale_after_softmax": ("            out[b, h] = p @ Vb[:, kvh, :]\n    return out",
                            "            out[b, h] = scale * (p @ Vb[:, kvh, :])\n    return out"),
    "scale_twice": ("            s = scale * (Kb[:, kvh, :] @ qf[b, h])",
                    "            s = scale * scale * (Kb[:, kvh, :] @ qf[b, h])"),
    "kv_swapped_in_decode": ("        Kb = stored_to_f64(gather_context(k_cache, block_tables[b], n), dtype)  #",
                             "        Kb = stored_to_f64(gather_context(v_cache, block_tables[b], n), dtype)  #"),
    "no_max_shift_normalisation": ("            p = e / e.sum()", "            p = e / e.max()"),
    "q_head_index": ("            s = scale * (Kb[:, kvh, :] @ qf[b, h])",
                     "            s = scale * (Kb[:, kvh, :] @ qf[b, kvh])"),
    "bf16_shift": ("<< np.uint32(16))", "<< np.uint32(15))"),
    "bf16_signed": ("    w = (b.astype(np.uint16).astype(np.uint32) << np.uint32(16))",
                    "    w = (b.astype(np.int16).astype(np.int32).astype(np.uint32) << np.uint32(17) >> np.uint32(1))"),
    # the page-2 fold
    "fold_no_correction": ("                    c = math.exp(m - m_new) if m != -math.inf else 0.0",
                           "                    c = 1.0"),
    "fold_sum_unscaled": ("                    l = l * c + p", "                    l = l + p"),
    "fold_off_by_one": ("                    if pos >= n:", "                    if pos > n:"),
    # prefill (causal varlen)
    "prefill_mask_excludes_self": ("        visible = np.arange(n)[None, :] <= pos[:, None]",
                                   "        visible = np.arange(n)[None, :] < pos[:, None]"),
    "prefill_no_mask": ("            s = np.where(visible, s, -np.inf)\n", ""),
    "prefill_top_left_alignment": ("    return np.arange(n - num_queries, n, dtype=np.int64)",
                                   "    return np.arange(0, num_queries, dtype=np.int64)"),
    "prefill_query_rows_shifted": ("            s = scale * (qf[s0:s1, h, :] @ Kb[:, kvh, :].T)",
                                   "            s = scale * (qf[s0 + (s1 - s0 > 1):s1 + (s1 - s0 > 1), h, :] @ Kb[:, kvh, :].T)"),
    "prefill_kv_head_mod": ("        for h in range(H):\n            kvh = kv_head_of(h, H, KVH)\n            s = scale * (qf[s0:s1",
                            "        for h in range(H):\n            kvh = h % KVH\n            s = scale * (qf[s0:s1"),
    "prefill_scale_dropped": ("            s = scale * (qf[s0:s1, h, :] @ Kb[:, kvh, :].T)",
                              "            s = (qf[s0:s1, h, :] @ Kb[:, kvh, :].T)"),
    "prefill_softmax_over_queries": ("            p = e / e.sum(axis=1, keepdims=True)",
                                     "            p = e / e.sum(axis=0, keepdims=True)"),
    # vLLM cache layout
    "vllm_k_token_and_group_swapped": ("reshape(NB, bs, KVH, D // x, x).transpose(0, 2, 3, 1, 4)",
                                       "reshape(NB, bs, KVH, D // x, x).transpose(0, 2, 1, 3, 4)"),
    "vllm_pack_width_elements": ('    return {"bf16": 8, "f32": 4}[dtype]', '    return {"bf16": 8, "f32": 8}[dtype]'),
    "vllm_v_not_transposed": ("    return np.ascontiguousarray(v_cache.transpose(0, 2, 3, 1))",
                              "    return np.ascontiguousarray(v_cache.transpose(0, 2, 1, 3))"),
    "prefill_v_from_k": ("            out[s0:s1, h] = p @ Vb[:, kvh, :]", "            out[s0:s1, h] = p @ Kb[:, kvh, :]"),
}


def _mutant(name):
    src = open(SRC, encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    O = _mutant(name)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (Exception, pytest.fail.Exception) as e:  # noqa: BLE001 - any failure counts
            failures.append((pin.__name__, type(e).__name__))
    assert failures, f"no pin catches mutant {name}"
