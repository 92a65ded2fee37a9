"""Sliding-window attention through the C ABI, against the fp64 oracle:
prefill, chunked prefill against a paged cache, and decode.

Tolerances as for every attention output (fp32 max-abs 1e-5; bf16 max-abs
2e-2 and mean-abs 2e-3; LSE 1e-4).  Blocks that lie wholly before every
window of a call are never read: the tests mark them -1 in the block table
(as a cache that released them would) and expect the same bits.
"""
import math
import sys

import numpy as np
import pytest
import torch

import full_size as FS
import oracle
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max=1e-5, mean=1e-5), "bf16": dict(max=2e-2, mean=2e-3)}
LSE_TOL = 1e-4
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check(o_gpu, lse_gpu, O_ref, lse_ref, dt, what=""):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    assert O.shape == np.asarray(O_ref).shape
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    assert err.max() <= TOL[dt]["max"], f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= TOL[dt]["mean"], f"{what}: mean abs err {err.mean():.3e}"
    L = lse_gpu.detach().to("cpu", torch.float64).numpy()
    e = np.abs(L - lse_ref).max()
    assert e <= LSE_TOL, f"{what}: LSE err {e:.3e}"


def evict_before_window(table, seq_lens, bs, first_key):
    """Copy of the table with -1 for every block wholly before first_key(b)."""
    t = table.clone()
    for b, L in enumerate(seq_lens.tolist()):
        n = first_key(b, L) // bs
        t[b, :n] = -1
    return t


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------
PREFILL_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, window
    (1, 2, 1, 6, 6, 64, 3),            # the printed window-3 mask's shape
    (2, 4, 2, 200, 200, 128, 1),
    (1, 4, 2, 300, 300, 128, 64),
    (1, 8, 2, 383, 383, 128, 100),
    (1, 4, 1, 257, 257, 64, 129),
    (1, 4, 2, 70, 333, 128, 90),       # queries extend a cache: bottom-right
    (2, 2, 2, 520, 520, 64, 256),
    (1, 4, 2, 1100, 1100, 128, 300),   # nine 128-position query tiles (2 heads each) in pairs
    (1, 8, 2, 700, 700, 128, 200),     # eleven 64-position tiles (4 heads each); waves start their windows tiles apart
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_W{}".format(*c))
def test_window_prefill_small(fa, case, dt):
    B, Hq, Hkv, Nq, Nk, d, Wn = case
    note(f"window prefill {dt} {case}")
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed=500 + Wn + Nq)
    scale = 1 / math.sqrt(d)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=scale, window=Wn)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.prefill(q, k, v, scale, True, window=Wn)
    check(o, lse, O_ref, lse_ref, dt, f"window prefill {case}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_window_covering_everything_is_causal(fa, dt):
    """A window as long as the sequence, or longer, is plain causal attention.
    In fp32 one kernel serves both, bit for bit.  In bf16 the windowed
    instance takes each tile's row max before its weights, while the causal one
    checks the weights afterwards, so the two use different references and
    round differently. They agree within one bf16 rounding of the output
    (2^-7 relative bounds it) and 1e-5 on the LSE, and each matches the oracle.
    The two windows give the same bits."""
    q, k, v = W.make_prefill_inputs(1, 8, 2, 300, 300, 128, dt, seed=9)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o0, l0 = fa.prefill(qd, kd, vd, causal=True)
    o1, l1 = fa.prefill(qd, kd, vd, causal=True, window=300)
    o2, l2 = fa.prefill(qd, kd, vd, causal=True, window=10_000)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(l1), bits(l2))
    if dt == "f32":
        assert torch.equal(bits(o0), bits(o1)) and torch.equal(bits(l0), bits(l1))
    else:
        a, b = o0.double().cpu(), o1.double().cpu()
        assert ((a - b).abs() <= 2.0 ** -7 * torch.maximum(a.abs(), b.abs())).all()
        assert (l0.double() - l1.double()).abs().max().item() <= 1e-5
    O_ref, lse_ref = oracle.prefill(q, k, v, 1 / math.sqrt(128), True)
    check(o0, l0, O_ref, lse_ref, dt, "causal")
    check(o1, l1, O_ref, lse_ref, dt, "window 300")


# ----------------------------------------------------------------------------
# chunked prefill against a paged cache
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("bs", [16, 4])
def test_window_chunked_prefill(fa, dt, bs):
    Wn, n = 100, 70
    ci = W.make_chunked_inputs(3, 4, 2, 128, dt, seed=600 + bs, chunk=n, past_lens=[300, 10, 129], block_size=bs)
    kc, vc = ci.k_cache.to(DEV), ci.v_cache.to(DEV)
    lens, table = ci.seq_lens.to(DEV), ci.block_table.to(DEV)
    fa.kv_append(ci.k_new.to(DEV), ci.v_new.to(DEV), kc, vc, lens, block_table=table)
    q = ci.q.to(DEV)
    o, lse = fa.chunked_prefill(q, kc, vc, lens, block_table=table, max_seq_len=ci.max_seq_len, window=Wn)
    # blocks before the chunk's first window are never read
    ev = evict_before_window(ci.block_table, ci.seq_lens, bs, lambda b, L: max(0, L - n - Wn + 1))
    o2, lse2 = fa.chunked_prefill(q, kc, vc, lens, block_table=ev.to(DEV), max_seq_len=ci.max_seq_len, window=Wn)
    torch.cuda.synchronize()
    assert torch.equal(bits(o), bits(o2)) and torch.equal(bits(lse), bits(lse2))
    kr, vr = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, bs)
    O_ref, lse_ref = oracle.chunked_prefill(ci.q, kr, vr, ci.seq_lens, 1 / math.sqrt(128), True,
                                            ci.block_table, bs, window=Wn)
    check(o, lse, O_ref, lse_ref, dt, "window chunked prefill")


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # B, Hq, Hkv, d, lens, paged, bs, window, split_tokens
    (4, 8, 2, 128, [1, 50, 64, 1000], True, 16, 64, 0),
    (4, 8, 2, 128, [1, 50, 300, 3000], True, 16, 700, 256),     # several splits inside the window
    (3, 4, 4, 64, [5, 129, 2000], True, 1, 129, 256),
    (3, 32, 8, 128, [100, 4096, 9000], True, 16, 4096, 0),
    (3, 8, 1, 128, [7, 700, 1500], False, 0, 512, 256),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_{}_bs{}_W{}_st{}".format(
    c[0], c[1], c[2], c[3], "paged" if c[5] else "contig", c[6], c[7], c[8]))
def test_window_decode(fa, case, dt):
    B, Hq, Hkv, d, lens, paged, bs, Wn, st = case
    note(f"window decode {dt} {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, dt, seed=700 + Wn, seq_lens=lens, paged=paged, block_size=max(bs, 1))
    scale = 1 / math.sqrt(d)
    args = dict(max_seq_len=di.max_seq_len, scale=scale, split_tokens=st, window=Wn)
    q, kc, vc, sl = di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV)
    table = di.block_table.to(DEV) if paged else None
    o, lse = fa.decode(q, kc, vc, sl, block_table=table, **args)
    if paged:
        ev = evict_before_window(di.block_table, di.seq_lens, bs, lambda b, L: max(0, L - Wn))
        o2, lse2 = fa.decode(q, kc, vc, sl, block_table=ev.to(DEV), **args)
    torch.cuda.synchronize()
    if paged:
        assert torch.equal(bits(o), bits(o2)) and torch.equal(bits(lse), bits(lse2))
        O_ref, lse_ref = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, bs, scale,
                                             window=Wn)
    else:
        O_ref, lse_ref = oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, scale, window=Wn)
    check(o, lse, O_ref, lse_ref, dt, f"window decode {case}")


# ----------------------------------------------------------------------------
# full-size windowed workloads, in the launch configuration the benchmark times
# ----------------------------------------------------------------------------
def test_window_prefill_full_size(fa):
    """N = 32768 with a 4096-key window: every row of one query head per KV
    head against the oracle, plus rows sampled over all heads."""
    w = W.WINDOW_PREFILL
    note(f"window prefill {w.name}")
    q, k, v = W.prefill_inputs(w)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, scale=w.scale, window=w.window)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    del o, lse
    assert torch.isfinite(o_c.float()).all() and torch.isfinite(lse_c).all()
    n_rep = w.Hq // w.Hkv
    heads = [(0, g * n_rep + g % n_rep) for g in range(w.Hkv)]
    note(f"window prefill: oracle over heads {heads}")
    ref = FS.prefill_heads(q, k, v, w.scale, True, heads, window=w.window)
    for b, h in heads:
        check(o_c[b, h], lse_c[b, h], ref[(b, h)][0], ref[(b, h)][1], "bf16", f"window prefill head {h}")
    rng = np.random.default_rng(11)
    rows = [(0, int(rng.integers(w.Hq)), i) for i in (0, 1, 127, 128, w.window - 1, w.window, w.window + 63,
                                                       w.Nq - 129, w.Nq - 1)]
    rows += [(0, int(rng.integers(w.Hq)), int(rng.integers(w.Nq))) for _ in range(23)]
    O_ref, lse_ref = oracle.prefill_rows(q, k, v, w.scale, True, rows, window=w.window)
    idx = tuple(torch.tensor(c) for c in zip(*rows))
    check(o_c[idx], lse_c[idx], O_ref, lse_ref, "bf16", "window prefill rows")


def test_window_decode_full_size(fa):
    """The windowed decode batch: every (sequence, head) output and LSE."""
    w = W.WINDOW_DECODE
    note(f"window decode {w.name}")
    di = W.decode_inputs(w)
    o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                       block_table=di.block_table.to(DEV), max_seq_len=di.max_seq_len, scale=w.scale,
                       window=w.window)
    torch.cuda.synchronize()
    note("window decode: oracle over the whole batch")
    O_ref, lse_ref = FS.decode_batches(
        lambda heads: oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens,
                                          w.block_size, w.scale, heads=heads, window=w.window), w.B, w.Hq)
    check(o.cpu(), lse.cpu(), O_ref, lse_ref, "bf16", "window decode, every output")
