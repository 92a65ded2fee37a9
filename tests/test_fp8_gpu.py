"""FP8 (E4M3) KV cache through the C ABI, against the fp64 oracle.

The quantising append must give the oracle's codes bit for bit (a NaN input
only has to stay NaN); decode against an FP8 cache uses the bf16 tolerances
(max-abs 2e-2, mean-abs 2e-3; LSE 1e-4) against the oracle's decode over the
decoded cache values.
"""
import math
import sys

import numpy as np
import pytest
import torch

import full_size as FS
import oracle
from oracle import fp8 as F
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = dict(max=2e-2, mean=2e-3)
LSE_TOL = 1e-4
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(o_gpu, lse_gpu, O_ref, lse_ref, what=""):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    assert O.shape == np.asarray(O_ref).shape
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    assert err.max() <= TOL["max"], f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= TOL["mean"], f"{what}: mean abs err {err.mean():.3e}"
    L = lse_gpu.detach().to("cpu", torch.float64).numpy()
    e = np.abs(L - lse_ref).max()
    assert e <= LSE_TOL, f"{what}: LSE err {e:.3e}"


# ----------------------------------------------------------------------------
# the quantising append
# ----------------------------------------------------------------------------
def _append_case(B, Hkv, d, n, past, bs, ks, vs, k_new=None, v_new=None, seed=0):
    # an FP8 pool whose past slots hold codes and whose other slots hold NaN codes
    di = W.make_decode_inputs(B, 2 * Hkv, Hkv, d, "fp8", seed, seq_lens=[p + n for p in past], paged=True,
                              block_size=bs, spare_blocks=1)
    kc, vc = di.k_cache.clone(), di.v_cache.clone()
    for b, p in enumerate(past):
        for t in range(p, p + n):
            kc[int(di.block_table[b, t // bs]), t % bs] = W.FP8_NAN
            vc[int(di.block_table[b, t // bs]), t % bs] = W.FP8_NAN
    g = torch.Generator().manual_seed(seed + 1)
    if k_new is None:
        k_new = (torch.randn(B, Hkv, n, d, generator=g) * 3).to(torch.bfloat16)
    if v_new is None:
        v_new = (torch.randn(B, Hkv, n, d, generator=g) * 3).to(torch.bfloat16)
    return di, kc, vc, k_new, v_new


def _run_append(fa, di, kc, vc, k_new, v_new, ks, vs):
    kg, vg = kc.to(DEV), vc.to(DEV)
    fa.kv_append_fp8(k_new.to(DEV), v_new.to(DEV), kg, vg, di.seq_lens.to(DEV), ks, vs,
                     block_table=di.block_table.to(DEV))
    torch.cuda.synchronize()
    kr, vr = F.append_fp8(kc, vc, di.block_table, di.seq_lens, k_new, v_new, di.block_size, ks, vs)
    return kg.cpu().numpy(), vg.cpu().numpy(), kr, vr


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (1 / 64, 0.02), (0.37, 3.0)])
def test_append_fp8_random_values_bit_exact(fa, ks, vs):
    di, kc, vc, kn, vn = _append_case(3, 2, 128, 37, [0, 20, 16], 16, ks, vs, seed=int(ks * 100))
    kn, vn = (kn.float() * ks).to(torch.bfloat16), (vn.float() * vs).to(torch.bfloat16)
    kg, vg, kr, vr = _run_append(fa, di, kc, vc, kn, vn, ks, vs)
    assert np.array_equal(kg, kr) and np.array_equal(vg, vr)


def test_append_fp8_ties_saturation_signed_zero_and_nan(fa):
    """Exact midpoints between neighbouring E4M3 values (they must go to the
    even code), values beyond 448 (saturate), -0.0, and NaN."""
    s = 0.25                                               # a power of two: x / s is exact
    vals = F.decode_codes(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2                      # 126 ties, exact in bf16
    special = np.array([449.0, 464.0, 1e4, -1e4, -0.0, 0.0, np.nan, -np.nan])
    row = np.concatenate([mids, -mids, special])
    d = 128
    n = (len(row) + d - 1) // d
    x = np.full(n * d, 1.0)
    x[:len(row)] = row
    k_new = torch.tensor(x * s, dtype=torch.float64).to(torch.bfloat16).view(1, 1, n, d)
    assert np.array_equal(k_new.double().numpy().ravel()[:len(mids)] / s, mids)   # ties survive bf16
    di, kc, vc, _, _ = _append_case(1, 1, d, n, [5], 4, s, s, seed=3)
    kg, vg, kr, vr = _run_append(fa, di, kc, vc, k_new, k_new.clone(), s, s)
    for got, ref in ((kg, kr), (vg, vr)):
        nan_ref = np.isnan(F.decode_codes(ref))
        assert np.array_equal(np.isnan(F.decode_codes(got)), nan_ref)
        assert np.array_equal(np.where(nan_ref, 0, got), np.where(nan_ref, 0, ref))


# ----------------------------------------------------------------------------
# decode against an FP8 cache
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # B, Hq, Hkv, d, lens, paged, bs, split_tokens, window
    (3, 8, 2, 128, [1, 17, 700], True, 16, 256, 0),
    (3, 32, 8, 128, [200, 1000, 3000], True, 16, 0, 0),
    (2, 4, 4, 64, [129, 2000], True, 4, 512, 0),
    (4, 8, 1, 128, [3, 64, 65, 1500], False, 0, 256, 0),
    (3, 16, 2, 64, [10, 300, 2500], True, 16, 256, 700),
    (2, 8, 8, 128, [4096, 5000], True, 32, 0, 0),
    # a window over 4-token blocks, 1-token blocks with 16 query heads per KV head, and
    # sequences shorter than one stage
    (2, 16, 4, 128, [33, 2500], True, 4, 512, 300),
    (3, 16, 1, 128, [1, 129, 1000], True, 1, 256, 0),
    (3, 8, 2, 128, [31, 32, 5], False, 0, 256, 0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_{}_bs{}_st{}_W{}".format(
    c[0], c[1], c[2], c[3], "paged" if c[5] else "contig", c[6], c[7], c[8]))
def test_decode_fp8_small(fa, case):
    B, Hq, Hkv, d, lens, paged, bs, st, Wn = case
    note(f"fp8 decode {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, "fp8", seed=900 + d + B, seq_lens=lens, paged=paged,
                              block_size=max(bs, 1))
    scale = 1 / math.sqrt(d)
    ks, vs = W.FP8_SCALE, W.FP8_SCALE * 0.5
    table = di.block_table.to(DEV) if paged else None
    o, lse = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), ks, vs,
                           block_table=table, max_seq_len=di.max_seq_len, scale=scale, split_tokens=st, window=Wn)
    torch.cuda.synchronize()
    O_ref, lse_ref = F.decode_fp8(di.q, di.k_cache, di.v_cache, di.seq_lens, scale, ks, vs,
                                  di.block_table if paged else None, di.block_size, window=Wn)
    check(o, lse, O_ref, lse_ref, f"fp8 decode {case}")


def test_decode_fp8_reads_float8_tensors_too(fa):
    di = W.make_decode_inputs(2, 8, 2, 128, "fp8", 31, seq_lens=[40, 300], paged=True)
    args = dict(block_table=di.block_table.to(DEV), max_seq_len=di.max_seq_len)
    lens = di.seq_lens.to(DEV)
    o1, l1 = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), lens, 0.5, 0.5, **args)
    o2, l2 = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV).view(torch.float8_e4m3fn),
                           di.v_cache.to(DEV).view(torch.float8_e4m3fn), lens, 0.5, 0.5, **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_fp8_flags_invalid_device_inputs_with_nan(fa):
    di = W.make_decode_inputs(3, 8, 2, 128, "fp8", 32, seq_lens=[50, 50, 50], paged=True)
    lens = di.seq_lens.clone()
    lens[0] = di.max_seq_len + 1
    table = di.block_table.clone()
    table[1, 2] = di.kv_capacity + 5
    o, lse = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), lens.to(DEV), 1 / 64, 1 / 64,
                           block_table=table.to(DEV), max_seq_len=di.max_seq_len)
    torch.cuda.synchronize()
    o, lse = o.float().cpu(), lse.cpu()
    assert torch.isnan(o[:2]).all() and torch.isnan(lse[:2]).all()
    O_ref, lse_ref = F.decode_fp8(di.q[2:], di.k_cache, di.v_cache, di.seq_lens[2:], 1 / math.sqrt(128), 1 / 64,
                                  1 / 64, di.block_table[2:], 16)
    check(o[2:], lse[2:], O_ref, lse_ref, "valid sequence next to invalid ones")


def test_append_then_decode_fp8(fa):
    """A decode step as a server runs it: quantise the new token's K/V into the
    FP8 cache, then attend against it."""
    di = W.make_decode_inputs(4, 8, 2, 128, "fp8", 33, seq_lens=[1, 30, 257, 1000], paged=True)
    g = torch.Generator().manual_seed(34)
    kn = (torch.randn(4, 2, 1, 128, generator=g)).to(torch.bfloat16)
    vn = (torch.randn(4, 2, 1, 128, generator=g)).to(torch.bfloat16)
    kc, vc = di.k_cache.to(DEV), di.v_cache.to(DEV)
    lens, table = di.seq_lens.to(DEV), di.block_table.to(DEV)
    fa.kv_append_fp8(kn.to(DEV), vn.to(DEV), kc, vc, lens, W.FP8_SCALE, W.FP8_SCALE, block_table=table)
    o, lse = fa.decode_fp8(di.q.to(DEV), kc, vc, lens, W.FP8_SCALE, W.FP8_SCALE, block_table=table,
                           max_seq_len=di.max_seq_len, split_tokens=256)
    torch.cuda.synchronize()
    kr, vr = F.append_fp8(di.k_cache, di.v_cache, di.block_table, di.seq_lens, kn, vn, 16, W.FP8_SCALE,
                          W.FP8_SCALE)
    assert np.array_equal(kc.cpu().numpy(), kr) and np.array_equal(vc.cpu().numpy(), vr)
    O_ref, lse_ref = F.decode_fp8(di.q, kr, vr, di.seq_lens, 1 / math.sqrt(128), W.FP8_SCALE, W.FP8_SCALE,
                                  di.block_table, 16)
    check(o, lse, O_ref, lse_ref, "append then decode")


def test_fp8_decode_full_size(fa):
    """The FP8 decode batch in the benchmark's launch configuration: every
    (sequence, head) output and LSE against the oracle."""
    w = W.FP8_DECODE
    note(f"fp8 decode {w.name}")
    di = W.decode_inputs(w)
    o, lse = fa.decode_fp8(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                           W.FP8_SCALE, W.FP8_SCALE, block_table=di.block_table.to(DEV),
                           max_seq_len=di.max_seq_len, scale=w.scale)
    torch.cuda.synchronize()
    note("fp8 decode: oracle over the whole batch")
    O_ref, lse_ref = FS.decode_batches(
        lambda heads: F.decode_fp8(di.q, di.k_cache, di.v_cache, di.seq_lens, w.scale, W.FP8_SCALE, W.FP8_SCALE,
                                   di.block_table, w.block_size, heads=heads), w.B, w.Hq)
    check(o.cpu(), lse.cpu(), O_ref, lse_ref, "fp8 decode, every output")
