"""Precision of the probabilities in the bf16 decode's P.V product, isolated.

"P09 · Paged KV 写入 + decode attention" (L3 详解) takes q, k and v to fp32
for the scores, the softmax and the weighted sum; its 易错点 puts a softmax
done in bf16 at about 1e-2 from the fp32 result.  The matrix-core kernel
carries each probability into the P.V product as a pair of bf16 values whose
sum is the fp32 probability to about 2^-17, so the weighted sum is fp32's.

The output itself is rounded to bf16, which hides that term, so this test
reads the fp32 partial results the partial kernel leaves in the workspace
(pa_decode_partials; layout in the header): for partition p, acc / l is the
softmax-weighted V over the partition's tokens alone, which is the oracle's
decode over exactly those tokens (the partition is whole blocks of the table
row).  Inputs: the long-context workload's longest sequence (128 partitions
of 1024 tokens), as drawn, with q scaled up (peaked attention: a few tokens
carry most of the weight) and with q scaled down (near-uniform weights, where
a rounding of P with the same sign everywhere would be systematic).

For each input the test reports the largest error of the GPU's partials and
of a host emulation of the kernel with P rounded to bf16 (round to nearest
even, the sum l still over fp32 values), and requires the GPU's to be ten
times smaller than the emulation's and below 1e-4 + 1e-4 |ref|.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O
import paged_kv_cache_70_amd as pk
from synth import CONFIGS, make_workload, stored_np
from tests.gpu_util import assert_matches_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    pk.load_library()
    yield


def _say(msg):
    print(f"[precision] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def longest():
    w = make_workload(CONFIGS["long_ctx_bf16"], "cuda")
    lens = stored_np(w.context_lens)
    b = int(np.argmax(lens))
    return w, b, int(lens[b])


def _bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest even) -> fp64, via torch's casts."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("q_gain", [1.0, 16.0, 0.02], ids=["as_drawn", "peaked", "near_uniform"])
def test_partials_carry_fp32_probabilities(longest, q_gain):
    w, b, n = longest
    H, D = w.q.shape[1], w.q.shape[2]
    KVH, bs = w.k_cache.shape[2], w.k_cache.shape[1]
    G = H // KVH
    q = (w.q[b:b + 1].float() * q_gain).to(torch.bfloat16).contiguous()
    tbl = w.block_tables[b:b + 1].contiguous()
    ctx = w.context_lens[b:b + 1].contiguous()
    W = tbl.shape[1]
    P = pk.partition_size(1, H, W, w.k_cache)
    maxP = -(-W * bs // P)
    ws = pk.new_workspace(1, H, W, w.k_cache, P)
    out = torch.empty_like(q)
    pk.decode_partials(q, w.k_cache, w.v_cache, tbl, ctx, w.scale, out=out, workspace=ws, partition_size=P)
    pk.decode_merge(q, w.k_cache, tbl, ctx, out=out, workspace=ws, partition_size=P)
    torch.cuda.synchronize()
    nacc = H * maxP * D
    wsf = ws.view(torch.float32)
    acc = wsf[:nacc].view(H, maxP, D).double().cpu().numpy()
    ml = wsf[nacc:nacc + H * maxP * 2].view(H, maxP, 2).double().cpu().numpy()
    npart = -(-n // P)
    assert npart > 1
    kc, vc = stored_np(w.k_cache), stored_np(w.v_cache)
    qn, tn = stored_np(q), stored_np(tbl)
    gpu_err = emu_err = 0.0
    worst_ok = 0.0
    for p in range(npart):
        t0, t1 = p * P, min(n, (p + 1) * P)
        sub_tbl = tn[:, t0 // bs:]
        ref = O.decode(qn, kc, vc, sub_tbl, np.array([t1 - t0], dtype=np.int32), w.scale, "bf16")[0]   # [H, D]
        part = acc[:, p, :] / ml[:, p, 1:2]
        e = np.abs(part - ref)
        gpu_err = max(gpu_err, float(e.max()))
        worst_ok = max(worst_ok, float((e / (1e-4 + 1e-4 * np.abs(ref))).max()))
        # host emulation of bf16-rounded P (fp32 probabilities rounded to nearest even)
        K = O.stored_to_f64(O.gather_context(kc, sub_tbl[0], t1 - t0), "bf16")     # [t, KVH, D]
        V = O.stored_to_f64(O.gather_context(vc, sub_tbl[0], t1 - t0), "bf16")
        qf = O.stored_to_f64(qn[0], "bf16")
        for h in range(H):
            s = w.scale * (K[:, h // G, :] @ qf[h])
            pr = np.exp(s - s.max()).astype(np.float32).astype(np.float64)
            emu = (_bf16_round(pr) @ V[:, h // G, :]) / pr.sum()
            emu_err = max(emu_err, float(np.abs(emu - ref[h]).max()))
    _say(f"q x {q_gain}: sequence {b} (n={n}, {npart} partitions of {P}): max |partial - oracle| "
         f"{gpu_err:.2e} with hi+lo P; {emu_err:.2e} with P rounded to bf16 (host emulation)")
    assert worst_ok <= 1.0, f"partials off by more than 1e-4 + 1e-4|ref| (worst ratio {worst_ok:.2f})"
    assert gpu_err * 10 <= emu_err, (gpu_err, emu_err)
    ref_out = O.decode(qn, kc, vc, tn, stored_np(ctx), w.scale, "bf16")
    assert_matches_oracle(out, ref_out, "bf16", f"q x {q_gain}: merged output")
