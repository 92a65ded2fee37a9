"""Parity with the fp64 oracle on seeded random shapes, through the C ABI.

The hand-picked cases in the other parity files cover the known edges; these
draw head counts, GQA ratios, lengths, block sizes, split sizes, windows and
dtypes from a fixed seed, so that combinations nobody picked are exercised
too.  Every case is deterministic and named by its shape.  Tolerances as for
every attention output: fp32 max-abs 1e-5; bf16 max-abs 2e-2 and mean-abs
2e-3; LSE 1e-4 (rows with no visible key: O = 0 and LSE = -inf on both
sides).
"""
import math
import random
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from oracle import mla as M
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3)}
LSE_TOL = 1e-4
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(o_gpu, lse_gpu, O_ref, lse_ref, dt, what):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    O_ref = np.asarray(O_ref)
    assert O.shape == O_ref.shape, (what, O.shape, O_ref.shape)
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    assert err.max() <= TOL[dt]["max"], f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= TOL[dt]["mean"], f"{what}: mean abs err {err.mean():.3e}"
    L = lse_gpu.detach().to("cpu", torch.float64).numpy()
    inf_ref = np.isneginf(lse_ref)
    assert (np.isneginf(L) == inf_ref).all(), f"{what}: -inf LSE rows differ"
    if (~inf_ref).any():
        e = np.abs(L[~inf_ref] - lse_ref[~inf_ref]).max()
        assert e <= LSE_TOL, f"{what}: LSE err {e:.3e}"


def _heads(r):
    hkv = r.choice([1, 1, 2, 2, 4, 8])
    rep = r.choice([1, 2, 3, 4, 8])
    while hkv * rep > 16:
        rep = max(1, rep // 2)
    return hkv * rep, hkv


def _group_heads(r):
    # query heads per KV head whose largest power-of-two divisor is 2, 4 or 8:
    # 2, 4 or 8 heads share a prefill workgroup, in 3 or more workgroups per tile
    hkv = r.choice([1, 2])
    return hkv * r.choice([6, 12, 16, 24, 32]), hkv


def _prefill_cases(n, seed, heads=None):
    heads = heads or _heads
    r = random.Random(seed)
    cases = []
    for _ in range(n):
        hq, hkv = heads(r)
        d = r.choice([64, 128])
        dt = "f32" if r.random() < 0.2 else "bf16"
        causal = r.random() < 0.7
        nk = r.randint(1, 600)
        nq = r.randint(1, nk) if causal else r.randint(1, 600)
        win = r.randint(1, nk) if causal and r.random() < 0.35 else 0
        cases.append((r.choice([1, 2]), hq, hkv, nq, nk, d, causal, win, dt))
    return cases


def _decode_cases(n, seed):
    r = random.Random(seed)
    cases = []
    for _ in range(n):
        hq, hkv = _heads(r)
        d = r.choice([64, 128])
        dt = "f32" if r.random() < 0.2 else "bf16"
        B = r.randint(1, 5)
        lens = [r.choice([0, r.randint(1, 64), r.randint(1, 1500)]) for _ in range(B)]
        paged = r.random() < 0.6
        bs = r.choice([1, 2, 4, 8, 16, 16, 32, 64, 128]) if paged else 0
        split = r.choice([0, 0, 256, 512, 768, 2048])
        win = r.randint(1, max(lens) + 5) if r.random() < 0.3 else 0
        cases.append((B, hq, hkv, d, tuple(lens), paged, bs, split, win, dt))
    return cases


def _chunk_cases(n, seed, heads=None):
    heads = heads or _heads
    r = random.Random(seed)
    cases = []
    for _ in range(n):
        hq, hkv = heads(r)
        d = r.choice([64, 128])
        dt = "f32" if r.random() < 0.2 else "bf16"
        B = r.randint(1, 3)
        nq = r.randint(1, 400)
        causal = r.random() < 0.8
        lens = [nq + r.randint(0, 700) for _ in range(B)]
        paged = r.random() < 0.7
        bs = r.choice([1, 4, 8, 16, 32, 64]) if paged else 0
        win = r.randint(1, max(lens)) if causal and r.random() < 0.3 else 0
        cases.append((B, hq, hkv, d, nq, tuple(lens), paged, bs, causal, win, dt))
    return cases


def _mla_cases(n, seed):
    r = random.Random(seed)
    cases = []
    for _ in range(n):
        B = r.randint(1, 4)
        Hq = r.choice([8, 16, 40, 64, 128, 144])
        lens = [r.choice([0, r.randint(1, 100), r.randint(1, 3000)]) for _ in range(B)]
        paged = r.random() < 0.7
        bs = r.choice([1, 4, 8, 16, 32, 64]) if paged else 0
        split = r.choice([0, 0, 32, 256, 640, 2048])
        cases.append((B, Hq, tuple(lens), paged, bs, split))
    return cases


PREFILL = _prefill_cases(24, 20261) + _prefill_cases(10, 20265, _group_heads)
DECODE = _decode_cases(24, 20262)
CHUNKED = _chunk_cases(16, 20263) + _chunk_cases(6, 20266, _group_heads)
FP8 = [c for c in _decode_cases(12, 20264)]
MLA = _mla_cases(16, 20265)


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_w{}_{}".format(
    *c[:6], "causal" if c[6] else "full", c[7], c[8]))
def test_random_prefill(fa, case):
    B, Hq, Hkv, Nq, Nk, d, causal, win, dt = case
    note(f"random prefill {case}")
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed=Nq * 7 + Nk + d)
    scale = 1 / math.sqrt(d)
    O_ref, lse_ref = oracle.prefill(q, k, v, scale, causal, window=win)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale, window=win)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case))


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_{}_{}_bs{}_st{}_w{}_{}".format(
    c[0], c[1], c[2], c[3], "-".join(map(str, c[4])), "paged" if c[5] else "contig", *c[6:]))
def test_random_decode(fa, case):
    B, Hq, Hkv, d, lens, paged, bs, split, win, dt = case
    note(f"random decode {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, dt, seed=sum(lens) % 991 + d, seq_lens=list(lens), paged=paged,
                              block_size=bs or 16, s_cap=max(max(lens), 1) + 3, spare_blocks=2 if paged else 0)
    scale = 1 / math.sqrt(d)
    if paged:
        O_ref, lse_ref = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, di.block_size,
                                             scale, window=win)
        o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                           block_table=di.block_table.to(DEV), max_seq_len=di.max_seq_len, split_tokens=split,
                           window=win)
    else:
        O_ref, lse_ref = oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, scale, window=win)
        o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                           max_seq_len=di.max_seq_len, split_tokens=split, window=win)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case))


@pytest.mark.parametrize("case", CHUNKED, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_n{}_{}_{}_bs{}_{}_w{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], "-".join(map(str, c[5])), "paged" if c[6] else "contig", c[7],
    "causal" if c[8] else "full", c[9], c[10]))
def test_random_chunked_prefill(fa, case):
    """The Nq newest tokens of each sequence against its whole cache, the cache
    written beforehand (its lengths count the new tokens)."""
    B, Hq, Hkv, d, nq, lens, paged, bs, causal, win, dt = case
    note(f"random chunked prefill {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, dt, seed=sum(lens) % 983 + nq, seq_lens=list(lens), paged=paged,
                              block_size=bs or 16, s_cap=max(lens) + 5, spare_blocks=2 if paged else 0)
    q, _, _ = W.make_prefill_inputs(B, Hq, 1, nq, 1, d, dt, seed=nq + d)
    scale = 1 / math.sqrt(d)
    table = di.block_table if paged else None
    O_ref, lse_ref = oracle.chunked_prefill(q, di.k_cache, di.v_cache, di.seq_lens, scale, causal,
                                            table, di.block_size if paged else 0, window=win)
    o, lse = fa.chunked_prefill(q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                                block_table=table.to(DEV) if paged else None, max_seq_len=di.max_seq_len,
                                causal=causal, scale=scale, window=win)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case))


@pytest.mark.parametrize("case", FP8, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_{}_{}_bs{}_st{}_w{}".format(
    c[0], c[1], c[2], c[3], "-".join(map(str, c[4])), "paged" if c[5] else "contig", *c[6:9]))
def test_random_fp8_decode(fa, case):
    """bf16 queries against an E4M3 cache (per-tensor scales)."""
    B, Hq, Hkv, d, lens, paged, bs, split, win, _ = case
    note(f"random fp8 decode {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, "fp8", seed=sum(lens) % 977 + d, seq_lens=list(lens), paged=paged,
                              block_size=bs or 16, s_cap=max(max(lens), 1) + 3, spare_blocks=2 if paged else 0)
    scale = 1 / math.sqrt(d)
    ks, vs = W.FP8_SCALE, W.FP8_SCALE * 0.75
    table = di.block_table if paged else None
    O_ref, lse_ref = F.decode_fp8(di.q, di.k_cache, di.v_cache, di.seq_lens, scale, ks, vs, table, di.block_size,
                                  window=win)
    o, lse = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), ks, vs,
                           block_table=table.to(DEV) if paged else None, max_seq_len=di.max_seq_len, scale=scale,
                           split_tokens=split, window=win)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, "bf16", str(case))


@pytest.mark.parametrize("case", MLA, ids=lambda c: "B{}_Hq{}_{}_{}_bs{}_st{}".format(
    c[0], c[1], "-".join(map(str, c[2])), "paged" if c[3] else "contig", c[4], c[5]))
def test_random_mla_decode(fa, case):
    """Absorbed-latent MLA decode (d_c = 512, d_r = 64) in latent space."""
    B, Hq, lens, paged, bs, split = case
    note(f"random mla decode {case}")
    mi = W.make_mla_inputs(B, Hq, 512, 64, sum(lens) % 971 + Hq, seq_lens=list(lens), paged=paged,
                           block_size=bs or 16, s_cap=None if paged else max(max(lens), 1) + 7,
                           spare_blocks=1 if paged else 0)
    scale = 1 / math.sqrt(128 + 64)
    table = mi.block_table if paged else None
    O_ref, lse_ref = M.mla_decode_latent(mi.q, mi.kv, mi.seq_lens, scale, 512, table, mi.block_size)
    o, lse = fa.mla_decode(mi.q.to(DEV), mi.kv.to(DEV), mi.seq_lens.to(DEV), scale,
                           block_table=table.to(DEV) if paged else None, max_seq_len=mi.max_seq_len,
                           split_tokens=split)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, "bf16", str(case))
