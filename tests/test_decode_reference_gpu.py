"""Decode (bf16, fp32 and FP8 caches, contiguous and paged) and MLA decode
through the C ABI, on keys built to move the running maximum, against the
fp64 oracle.

Random normal keys leave a row's reference (the running max of the streaming
softmax, "Li Hongyi, Machine Learning 2026", lecture "FlashAttention") almost
still after its first keys.  Here:

* a ramp: the query is +8 or -8 on one dimension (alternating heads) and key
  t is `step * t` there, so the scores of the + heads climb by `per64`
  natural-log units every 64 keys and keep raising the maximum inside every
  split, while the - heads see theirs fall;
* spikes: a few keys score about 140 natural-log units above the rest, so
  the first look at them against the old reference overflows 2^x.

In MLA decode the value is the first 512 numbers of each cache row, so the
ramp and the spikes sit on the position part (dimension 512), which only the
score reads.

Bars: bf16 and FP8 outputs max-abs 2e-2 + 2^-7 |O| elementwise (a peaked
softmax gives outputs the size of one value row, up to ~5, where two bf16
roundings are worth 2^-7 |O|), mean-abs 2e-3; fp32 outputs 1e-5; LSE 1e-4.
Scores of size S are formed in fp32 by every kernel and carry absolute
rounding of a few S * 2^-24 into every exponent and into the LSE, so the LSE
bar, and the fp32 output bars, scale by max(1, S / 8).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from oracle import mla as M
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3), "fp8": dict(max=2e-2, mean=2e-3)}
LSE_TOL = 1e-4


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(o_gpu, lse_gpu, O_ref, lse_ref, dt, what, smax):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    O_ref = np.asarray(O_ref)
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    f_lse = max(1.0, smax / 8)
    f = f_lse if dt == "f32" else 1.0
    err = np.abs(O - O_ref)
    # a peaked softmax hands a bf16 output the size of one value row (|O| up
    # to ~5 here), where two bf16 roundings (a split's partial, the output)
    # are worth up to 2^-7 |O|
    rel = 2.0 ** -7 if dt != "f32" else 0.0
    over = err - (TOL[dt]["max"] * f + rel * np.abs(O_ref))
    assert over.max() <= 0, f"{what}: max abs err {err.max():.3e} (x{f:.1f}, + 2^-7 |O| in bf16)"
    assert err.mean() <= TOL[dt]["mean"] * f, f"{what}: mean abs err {err.mean():.3e} (x{f:.1f})"
    L = lse_gpu.detach().to("cpu", torch.float64).numpy()
    lse_ref = np.asarray(lse_ref)
    assert np.isfinite(lse_ref).all()
    e = np.abs(L - lse_ref).max()
    assert e <= LSE_TOL * f_lse, f"{what}: LSE err {e:.3e} (x{f_lse:.1f})"


def token_positions(di, b):
    """(index tuple into the K cache for token t of sequence b, for all t < L)
    as a function of t, for both layouts (the head axis left whole)."""
    L = int(di.seq_lens[b])
    t = torch.arange(L)
    if di.block_table is None:
        return (b, slice(None), t)
    blk = di.block_table[b].to(torch.int64)[t // di.block_size]
    return (blk, t % di.block_size, slice(None))


def set_key_dim0(di, b, values):
    """K[token t of sequence b, every KV head, dimension 0] = values[t]."""
    idx = token_positions(di, b)
    if di.block_table is None:
        di.k_cache[idx[0], :, idx[2], 0] = values.to(di.k_cache.dtype)[None, :]
    else:
        di.k_cache[idx[0], idx[1], :, 0] = values.to(di.k_cache.dtype)[:, None]


def score_max_gqa(q, di, scale, key_values):
    """Largest |q . k| * scale given the dimension-0 key values (the other
    dimensions are random normal and add at most a few units)."""
    return float(q[..., 0].abs().max()) * float(max(v.abs().max() for v in key_values)) * scale + 8.0


# ----------------------------------------------------------------------------
# GQA decode, bf16 and fp32 caches
# ----------------------------------------------------------------------------
CASES = [
    # B, Hq, Hkv, d, lens, paged, bs, split_tokens
    (3, 8, 2, 128, [700, 2000, 129], True, 16, 256),
    (3, 8, 2, 128, [700, 2000, 129], True, 16, 0),
    (2, 16, 4, 64, [1500, 333], False, 0, 512),
    (2, 8, 8, 128, [3000, 64], False, 0, 0),
]


def _id(c):
    return "B{}_Hq{}_Hkv{}_d{}_{}_st{}".format(c[0], c[1], c[2], c[3], "paged" if c[5] else "contig", c[7])


def _inputs(case, dt, seed):
    B, Hq, Hkv, d, lens, paged, bs, st = case
    return W.make_decode_inputs(B, Hq, Hkv, d, dt, seed=seed, seq_lens=lens, paged=paged, block_size=max(bs, 1),
                                s_cap=max(lens) + 5)


def _run(fa, di, case, scale):
    st = case[7]
    table = di.block_table.to(DEV) if di.block_table is not None else None
    return fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), block_table=table,
                     max_seq_len=di.max_seq_len, scale=scale, split_tokens=st)


def _oracle(di, scale):
    if di.block_table is not None:
        return oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, di.block_size, scale)
    return oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, scale)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_decode_keys_that_keep_raising_the_max(fa, case, dt):
    note(f"decode ramp {dt} {case}")
    d = case[3]
    di = _inputs(case, dt, seed=1500 + d + len(case[4]))
    scale = 1 / math.sqrt(d)
    per64 = 3.0
    step = per64 / 64 / (8 * scale)
    sign = torch.ones(di.q.shape[1])
    sign[1::2] = -1
    di.q[:, :, 0] = (8 * sign).to(di.q.dtype)[None, :]
    ramps = []
    for b in range(di.q.shape[0]):
        vals = torch.arange(int(di.seq_lens[b]), dtype=torch.float32) * step
        set_key_dim0(di, b, vals)
        ramps.append(vals)
    O_ref, lse_ref = _oracle(di, scale)
    o, lse = _run(fa, di, case, scale)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, f"ramp {case}", score_max_gqa(di.q, di, scale, ramps))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_decode_key_spikes_past_the_exponent_range(fa, case, dt):
    note(f"decode spikes {dt} {case}")
    d = case[3]
    di = _inputs(case, dt, seed=1600 + d + len(case[4]))
    scale = 1 / math.sqrt(d)
    di.q[:, :, 0] = 4.0
    spikes = []
    for b in range(di.q.shape[0]):
        L = int(di.seq_lens[b])
        at = sorted({L // 3, L // 3 + 1, (2 * L) // 3, L - 1})
        idx = token_positions(di, b)
        if di.block_table is None:
            col = di.k_cache[b, 0, :L, 0].float().clone()
        else:
            col = di.k_cache[idx[0], idx[1], 0, 0].float().clone()
        col[at] = 400.0 if d == 128 else 280.0
        set_key_dim0(di, b, col)
        spikes.append(col)
    O_ref, lse_ref = _oracle(di, scale)
    o, lse = _run(fa, di, case, scale)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, f"spikes {case}", score_max_gqa(di.q, di, scale, spikes))


# ----------------------------------------------------------------------------
# FP8 cache
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["ramp", "spikes"])
@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contig"])
def test_decode_fp8_moving_max(fa, kind, paged):
    note(f"fp8 decode {kind} paged={paged}")
    B, Hq, Hkv, d = 3, 8, 2, 128
    di = W.make_decode_inputs(B, Hq, Hkv, d, "fp8", seed=1700 + paged, seq_lens=[900, 2500, 70], paged=paged,
                              block_size=16, s_cap=2505)
    scale = 1 / math.sqrt(d)
    ks, vs = 1.0, W.FP8_SCALE
    cols = []
    if kind == "ramp":
        step = 3.0 / 64 / (8 * scale)
        sign = torch.ones(Hq)
        sign[1::2] = -1
        di.q[:, :, 0] = (8 * sign).to(di.q.dtype)[None, :]
    else:
        di.q[:, :, 0] = 4.0
    for b in range(B):
        L = int(di.seq_lens[b])
        if kind == "ramp":
            vals = torch.arange(L, dtype=torch.float32) * step
        else:
            vals = torch.zeros(L)
            vals[[L // 4, L // 2, L - 1]] = 400.0
        codes = (vals / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        idx = token_positions(di, b)
        if paged:
            di.k_cache[idx[0], idx[1], :, 0] = codes[:, None]
        else:
            di.k_cache[b, :, :L, 0] = codes[None, :]
        cols.append(codes.view(torch.float8_e4m3fn).float() * ks)
    table = di.block_table.to(DEV) if paged else None
    o, lse = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), ks, vs,
                           block_table=table, max_seq_len=di.max_seq_len, scale=scale, split_tokens=512)
    torch.cuda.synchronize()
    O_ref, lse_ref = F.decode_fp8(di.q, di.k_cache, di.v_cache, di.seq_lens, scale, ks, vs,
                                  di.block_table if paged else None, di.block_size)
    check(o, lse, O_ref, lse_ref, "fp8", f"fp8 {kind} paged={paged}", score_max_gqa(di.q, di, scale, cols))


# ----------------------------------------------------------------------------
# MLA decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["ramp", "spikes"])
@pytest.mark.parametrize("split", [256, 0])
def test_mla_decode_moving_max(fa, kind, split):
    note(f"mla decode {kind} split={split}")
    B, Hq, d_c, d_r = 3, 32, 512, 64
    mi = W.make_mla_inputs(B, Hq, d_c, d_r, seed=1800 + split, seq_lens=[700, 2600, 90], paged=True, block_size=64)
    scale = 1 / math.sqrt(128 + 64)
    pos = d_c  # first position dimension: read by the score only
    if kind == "ramp":
        step = 3.0 / 64 / (8 * scale)
        sign = torch.ones(Hq)
        sign[1::2] = -1
        mi.q[:, :, pos] = (8 * sign).to(mi.q.dtype)[None, :]
    else:
        mi.q[:, :, pos] = 4.0
    top = 0.0
    for b in range(B):
        L = int(mi.seq_lens[b])
        t = torch.arange(L)
        blk = mi.block_table[b].to(torch.int64)[t // mi.block_size]
        if kind == "ramp":
            vals = t.float() * step
        else:
            vals = mi.kv[blk, t % mi.block_size, pos].float().clone()
            vals[[L // 3, L - 1]] = 400.0
        mi.kv[blk, t % mi.block_size, pos] = vals.to(mi.kv.dtype)
        top = max(top, float(vals.abs().max()))
    o, lse = fa.mla_decode(mi.q.to(DEV), mi.kv.to(DEV), mi.seq_lens.to(DEV), scale,
                           block_table=mi.block_table.to(DEV), max_seq_len=mi.max_seq_len, split_tokens=split)
    torch.cuda.synchronize()
    O_ref, lse_ref = M.mla_decode_latent(mi.q, mi.kv, mi.seq_lens, scale, d_c, block_table=mi.block_table,
                                         block_size=mi.block_size)
    smax = float(mi.q[..., pos].abs().max()) * top * scale + 8.0
    check(o, lse, O_ref, lse_ref, "bf16", f"mla {kind} split={split}", smax)
