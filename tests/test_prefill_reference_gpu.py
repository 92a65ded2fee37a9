"""Prefill and chunked prefill (through the C ABI) on scores built to move the
running maximum, against the fp64 oracle (bf16: max-abs 2e-2, mean-abs 2e-3;
fp32: 1e-5; LSE 1e-4; the fp32 bars and the LSE bar times max(1, S / 8) for
scores up to S in size).

The streaming softmax keeps a reference per row that the weights are taken
against ("Li Hongyi, Machine Learning 2026", lecture "FlashAttention": running
max, rescaling of earlier partials).  Random normal inputs leave it almost
still after a row's first tile, so these inputs move it on purpose:

* a ramp: along dimension 0, every query row is +8 or -8 (alternating rows)
  and key j is `step * j`, so half of the rows of every wave see their scores
  climb by `per_tile` (natural-log units) over each 64-key tile and keep
  raising their maximum, while the other half see them fall;
* spikes: a few keys whose score stands about 140 (d = 128) or 200 (d = 64)
  natural-log units above every other, far past where 2^x overflows fp32, so
  the first look at such a tile against the old reference overflows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3)}
LSE_TOL = 1e-4
DEV = "cuda"
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def score_max(q, k, scale):
    """Largest |score| over every (query, key) pair of every head (fp64;
    query head h reads KV head h // (Hq / Hkv); masks ignored)."""
    kk = k.double().repeat_interleave(q.shape[1] // k.shape[1], dim=1)
    return float((q.double() @ kk.transpose(-1, -2)).abs().max()) * scale


def check(o_gpu, lse_gpu, O_ref, lse_ref, dt, what, smax=0.0):
    """Scores of size S, formed in fp32 by both kernels, carry absolute
    rounding of a few S * 2^-24 into every exponent and into the LSE (the
    score itself, its scaling, the subtraction), so the LSE bar, and the fp32
    output bars, scale with S past S = 8 (the normal inputs' range)."""
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    O_ref = np.asarray(O_ref)
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    f_lse = max(1.0, smax / 8)
    f = f_lse if dt == "f32" else 1.0
    assert err.max() <= TOL[dt]["max"] * f, f"{what}: max abs err {err.max():.3e} (x{f:.1f})"
    assert err.mean() <= TOL[dt]["mean"] * f, f"{what}: mean abs err {err.mean():.3e} (x{f:.1f})"
    L = lse_gpu.detach().to("cpu", torch.float64).numpy()
    lse_ref = np.asarray(lse_ref)
    assert np.isfinite(lse_ref).all()
    e = np.abs(L - lse_ref).max()
    assert e <= LSE_TOL * f_lse, f"{what}: LSE err {e:.3e} (x{f_lse:.1f})"


def ramp(q, k, per_tile, d, dt):
    """Queries +-8 on dimension 0 (alternating rows), key j = step * j there,
    so that a +8 row's score grows by per_tile over 64 keys."""
    step = per_tile / 64 / (8 / math.sqrt(d))
    sign = torch.ones(q.shape[-2])
    sign[1::2] = -1
    q[..., 0] = (8 * sign).to(TORCH_DT[dt])
    k[..., 0] = (torch.arange(k.shape[-2], dtype=torch.float32) * step).to(TORCH_DT[dt])


def spikes(q, k, at, dt):
    q[..., 0] = 4.0
    for j in at:
        k[..., j, 0] = 400.0


RAMP_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, per_tile, window
    (1, 4, 2, 700, 700, 128, True, 12.0, 0),     # every tile raises the max of the + rows
    (1, 2, 1, 300, 300, 64, True, 12.0, 0),
    (1, 4, 2, 130, 600, 128, False, 3.0, 0),     # a slow climb: some tiles pass the check, some not
    (2, 2, 2, 520, 520, 128, True, 0.7, 0),      # gentle: the reference lags within its slack
    (1, 4, 2, 700, 700, 128, True, 12.0, 100),   # sliding window: rows gain their first key tile by tile
]


def _ramp_id(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_rise{}_W{}".format(*c[:6], "causal" if c[6] else "full", c[7], c[8])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", RAMP_CASES, ids=_ramp_id)
def test_prefill_scores_that_keep_raising_the_max(fa, case, dt):
    B, Hq, Hkv, Nq, Nk, d, causal, per_tile, window = case
    note(f"prefill ramp {dt} {case}")
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed=900 + Nk + d)
    ramp(q, k, per_tile, d, dt)
    scale = 1 / math.sqrt(d)
    O_ref, lse_ref = oracle.prefill(q, k, v, scale, causal, window=window)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, window=window)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case), score_max(q, k, scale))


SPIKE_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, spike keys
    (1, 4, 2, 700, 700, 128, True, [5, 100, 101, 450]),
    (1, 2, 1, 300, 300, 64, True, [70, 200]),
    (1, 4, 2, 64, 900, 128, False, [640, 899]),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", SPIKE_CASES, ids=lambda c: "Nq{}_Nk{}_d{}_{}".format(c[3], c[4], c[5],
                                                                                      "causal" if c[6] else "full"))
def test_prefill_score_spikes_past_the_exponent_range(fa, case, dt):
    B, Hq, Hkv, Nq, Nk, d, causal, at = case
    note(f"prefill spikes {dt} {case}")
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed=950 + Nk + d)
    spikes(q, k, at, dt)
    scale = 1 / math.sqrt(d)
    O_ref, lse_ref = oracle.prefill(q, k, v, scale, causal)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case), score_max(q, k, scale))


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contig"])
def test_chunked_prefill_scores_that_keep_raising_the_max(fa, paged):
    """The chunk's keys ramp (the cached past is random), so the reference
    moves inside the chunk, tile by tile, in both cache layouts."""
    B, Hq, Hkv, d, n = 2, 4, 2, 128, 600
    past = [300, 1000]
    ci = W.make_chunked_inputs(B, Hq, Hkv, d, "bf16", seed=977, chunk=n, past_lens=past, paged=paged,
                               block_size=16, s_cap=(max(past) + n + 5) if not paged else None)
    ramp(ci.q, ci.k_new, 12.0, d, "bf16")
    spikes_at = [n // 2]
    ci.k_new[..., spikes_at, 0] = 300.0
    kc, vc = ci.k_cache.to(DEV), ci.v_cache.to(DEV)
    lens = ci.seq_lens.to(DEV)
    table = ci.block_table.to(DEV) if paged else None
    fa.kv_append(ci.k_new.to(DEV), ci.v_new.to(DEV), kc, vc, lens, block_table=table)
    scale = 1 / math.sqrt(d)
    o, lse = fa.chunked_prefill(ci.q.to(DEV), kc, vc, lens, block_table=table, max_seq_len=ci.max_seq_len,
                                scale=scale)
    torch.cuda.synchronize()
    if paged:
        kr, vr = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new,
                                     ci.block_size)
    else:
        kr, vr = oracle.append_batch_contiguous(ci.k_cache, ci.v_cache, ci.seq_lens, ci.k_new, ci.v_new)
    O_ref, lse_ref = oracle.chunked_prefill(ci.q, kr, vr, ci.seq_lens, scale, True, ci.block_table, ci.block_size)
    # the largest scores are the chunk's own (the past keys are random normal)
    check(o, lse, O_ref, lse_ref, "bf16", f"chunked paged={paged}", score_max(ci.q, ci.k_new, scale))
