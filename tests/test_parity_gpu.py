"""Parity of the HIP kernels (through the C ABI) with the fp64 oracle.

Tolerances: fp32 inputs, max-abs 1e-5 on O; bf16 inputs with fp32 accumulation,
max-abs 2e-2 and mean-abs 2e-3 on O; LSE within 1e-4 (rows with no visible key
must give exactly O = 0 and LSE = -inf on both sides).

Small shapes compare every output element.  The full-size workloads run in
the launch configuration the benchmark times: the N = 4096 prefill and both
decode batches compare every output element and LSE; the N = 32768 prefill
compares every row of one query head per KV head (all query-tile pairs, every
KV head) plus rows sampled over all heads.
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


def dtype_name(t):
    return "f32" if t.dtype == torch.float32 else "bf16"


def check(o_gpu, lse_gpu, O_ref, lse_ref, dt, what=""):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    O_ref = np.asarray(O_ref)
    assert O.shape == O_ref.shape, (O.shape, O_ref.shape)
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    assert err.max() <= TOL[dt]["max"], f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= TOL[dt]["mean"], f"{what}: mean abs err {err.mean():.3e}"
    if lse_gpu is not None:
        L = lse_gpu.detach().to("cpu", torch.float64).numpy()
        lse_ref = np.asarray(lse_ref)
        inf_ref = np.isneginf(lse_ref)
        assert (np.isneginf(L) == inf_ref).all(), f"{what}: -inf LSE rows differ"
        if (~inf_ref).any():
            e = np.abs(L[~inf_ref] - lse_ref[~inf_ref]).max()
            assert e <= LSE_TOL, f"{what}: LSE err {e:.3e}"
    return err.max()


# ----------------------------------------------------------------------------
# prefill, small shapes, every element
# ----------------------------------------------------------------------------
PREFILL_CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 1, 1, 64, True),
    (2, 4, 4, 64, 64, 64, True),          # MHA, exactly one tile
    (2, 4, 2, 65, 65, 128, True),         # ragged by one
    (1, 4, 1, 130, 130, 128, True),       # MQA
    (1, 6, 3, 257, 257, 64, True),
    (1, 8, 2, 200, 200, 128, False),
    (2, 2, 1, 127, 300, 128, False),      # Nq != Nk
    (1, 4, 2, 70, 200, 128, True),        # chunked prefill, bottom-right mask
    (1, 4, 2, 1, 333, 64, True),          # a single new query against a cache
    (1, 2, 2, 383, 383, 128, True),       # two 256-position tiles (MHA), ragged
    # the bf16 kernel runs query tiles (256 rows: 256 / hw positions of hw
    # heads) in complementary pairs; an odd count leaves a lone middle tile:
    (1, 4, 2, 700, 700, 128, True),       # six 128-position tiles: three pairs
    (1, 2, 1, 1200, 1300, 64, True),      # ten 128-position tiles, bottom-right mask, d = 64
    (2, 2, 2, 520, 520, 128, False),      # three 256-position tiles: a pair plus the lone middle one, no mask
    (1, 4, 1, 300, 300, 128, True),       # five 64-position tiles: two pairs plus the lone middle one
    # B * Hkv a multiple of 8: workgroups placed KV-head-major per XCD
    (2, 16, 8, 700, 700, 128, True),      # two (sequence, KV head) groups per XCD, pairs + middle tile
    (3, 8, 8, 300, 300, 64, True),        # three groups per XCD, MHA
    # query heads of one KV head share a workgroup (hw = the largest power of
    # two dividing Hq / Hkv, at most 8): 256 / hw positions of hw heads each
    (1, 16, 1, 300, 300, 128, True),      # Hq/Hkv 16: 8 heads x 32 positions, two workgroups per tile
    (1, 12, 2, 333, 333, 128, True),      # Hq/Hkv 6: 2 heads x 128 positions, three workgroups per tile
    (2, 24, 2, 250, 260, 64, True),       # Hq/Hkv 12: 4 heads x 64 positions, bottom-right mask
    (1, 32, 8, 520, 520, 128, True),      # Hq/Hkv 4, B * Hkv = 8: per-XCD placement of 64-position tiles
    (2, 64, 4, 200, 200, 128, True),      # Hq/Hkv 16, B * Hkv = 8: per-XCD placement, two workgroups per group
    (1, 16, 2, 100, 130, 128, False),     # Hq/Hkv 8, no mask
    (1, 32, 1, 290, 290, 128, True),      # MQA with 32 heads: 8 heads x 32 positions, four workgroups per tile
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}".format(*c[:6], "causal" if c[6] else "full"))
def test_prefill_small(fa, case, dt):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    note(f"prefill {dt} {case}")
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dt, seed=hash(case) % 1000 + (dt == "f32"))
    scale = 1 / math.sqrt(d)
    O_ref, lse_ref = oracle.prefill(q, k, v, scale, causal)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_no_keys_gives_zero_and_minus_inf(fa, dt):
    q, k, v = W.make_prefill_inputs(1, 2, 1, 5, 0, 64, dt, seed=3)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=False)
    torch.cuda.synchronize()
    assert (o.cpu() == 0).all() and torch.isneginf(lse.cpu()).all()


def test_prefill_scale_and_deterministic(fa):
    q, k, v = W.make_prefill_inputs(1, 4, 2, 190, 190, 128, "bf16", seed=5)
    O_ref, lse_ref = oracle.prefill(q, k, v, 0.3, True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fa.prefill(qd, kd, vd, causal=True, scale=0.3)
    o2, l2 = fa.prefill(qd, kd, vd, causal=True, scale=0.3)
    torch.cuda.synchronize()
    check(o1, l1, O_ref, lse_ref, "bf16")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prepared_calls_match_direct_calls(fa):
    """``prepare=True`` checks and marshals a call once; calling it again only
    enqueues the kernels.  Three replays give the direct call's bits."""
    q, k, v = W.make_prefill_inputs(1, 8, 2, 300, 300, 128, "bf16", seed=15)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_ref, l_ref = fa.prefill(qd, kd, vd, causal=True)
    call, o, l = fa.prefill(qd, kd, vd, causal=True, prepare=True)
    di = W.make_decode_inputs(3, 8, 2, 128, "bf16", seed=16, seq_lens=[900, 5, 2000], paged=True)
    dargs = (di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV))
    dkw = dict(block_table=di.block_table.to(DEV), max_seq_len=di.max_seq_len, split_tokens=256)
    do_ref, dl_ref = fa.decode(*dargs, **dkw)
    dcall, do, dl = fa.decode(*dargs, prepare=True, **dkw)
    torch.cuda.synchronize()
    for _ in range(3):
        o.zero_(); l.zero_(); do.zero_(); dl.zero_()
        call()
        dcall()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
        assert torch.equal(do, do_ref) and torch.equal(dl, dl_ref)


def test_prefill_writes_nothing_outside_its_output(fa):
    B, Hq, Hkv, N, d = 1, 4, 2, 100, 128
    q, k, v = W.make_prefill_inputs(B, Hq, Hkv, N, N, d, "bf16", seed=6)
    n = B * Hq * N * d
    guard = 4096
    buf = torch.full((n + 2 * guard,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((B * Hq * N + 2 * guard,), 7.0, dtype=torch.float32, device=DEV)
    out = buf[guard:guard + n].view(B, Hq, N, d)
    lse = lbuf[guard:guard + B * Hq * N].view(B, Hq, N)
    fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (buf[:guard] == 7).all() and (buf[-guard:] == 7).all()
    assert (lbuf[:guard] == 7).all() and (lbuf[-guard:] == 7).all()


def test_prefill_decode_consistency_through_the_kernels(fa):
    """The pages' cache test on the GPU path: decode with L cached tokens equals
    row L-1 of the causal prefill, both checked against the oracle."""
    Hq, Hkv, N, d = 8, 2, 77, 128
    q, k, v = W.make_prefill_inputs(1, Hq, Hkv, N, N, d, "bf16", seed=8)
    o_pre, lse_pre = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    lens = torch.tensor([N], dtype=torch.int32)
    o_dec, lse_dec = fa.decode(q[:, :, N - 1].contiguous().to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV), max_seq_len=N)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.decode_contiguous(q[:, :, N - 1], k, v, lens, 1 / math.sqrt(d))
    check(o_dec, lse_dec, O_ref, lse_ref, "bf16", "decode")
    check(o_pre[:, :, N - 1], lse_pre[:, :, N - 1], O_ref, lse_ref, "bf16", "prefill last row")


# ----------------------------------------------------------------------------
# decode, small shapes, every element
# ----------------------------------------------------------------------------
DECODE_CASES = [
    # B, Hq, Hkv, d, lens, paged, block_size, split_tokens
    (3, 4, 4, 128, [1, 2, 3], False, 0, 0),
    (4, 8, 2, 128, [5, 300, 257, 1000], False, 0, 256),     # several splits + merge
    (4, 8, 2, 64, [5, 300, 257, 1000], False, 0, 0),
    (2, 16, 1, 128, [700, 33], False, 0, 256),               # MQA: 2 groups of 8 heads
    (3, 6, 2, 128, [129, 64, 600], False, 0, 512),           # n_rep 3
    (5, 8, 4, 128, [0, 17, 256, 512, 513], False, 0, 256),   # empty sequence, split edges
    (4, 8, 2, 128, [5, 300, 257, 1000], True, 16, 256),
    (4, 8, 2, 64, [40, 17, 8, 31], True, 16, 0),              # the pages' paging demo lengths
    (3, 32, 8, 128, [1, 999, 2049], True, 16, 1024),
    (3, 4, 2, 128, [7, 100, 64], True, 1, 256),               # block size 1
    (3, 4, 2, 128, [7, 100, 64], True, 4, 0),
    (3, 8, 8, 64, [300, 1, 1030], True, 64, 256),
    (2, 8, 2, 128, [0, 90], True, 16, 0),
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_{}_{}_bs{}_st{}".format(
    c[0], c[1], c[2], c[3], "-".join(map(str, c[4])), "paged" if c[5] else "contig", c[6], c[7]))
def test_decode_small(fa, case, dt):
    B, Hq, Hkv, d, lens, paged, bs, split = case
    note(f"decode {dt} {case}")
    di = W.make_decode_inputs(B, Hq, Hkv, d, dt, seed=sum(lens) % 997, seq_lens=lens, paged=paged,
                              block_size=bs or 16, s_cap=max(max(lens), 1) + 5, spare_blocks=3 if paged else 0)
    scale = 1 / math.sqrt(d)
    if paged:
        O_ref, lse_ref = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, di.block_size, scale)
        o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                           block_table=di.block_table.to(DEV), max_seq_len=di.max_seq_len, split_tokens=split)
    else:
        O_ref, lse_ref = oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, scale)
        o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV),
                           max_seq_len=di.max_seq_len, split_tokens=split)
    torch.cuda.synchronize()
    check(o, lse, O_ref, lse_ref, dt, str(case))


def test_decode_split_count_does_not_change_the_answer_beyond_tolerance(fa):
    di = W.make_decode_inputs(2, 8, 2, 128, "bf16", seed=11, seq_lens=[3000, 1777], paged=True)
    O_ref, lse_ref = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, 16, 128 ** -0.5)
    args = (di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV))
    outs = []
    for st in (256, 512, 1024, 4096):
        o, lse = fa.decode(*args, block_table=di.block_table.to(DEV), max_seq_len=3000, split_tokens=st)
        torch.cuda.synchronize()
        check(o, lse, O_ref, lse_ref, "bf16", f"split {st}")
        outs.append(o)
    o2, _ = fa.decode(*args, block_table=di.block_table.to(DEV), max_seq_len=3000, split_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], o2)  # deterministic


def test_decode_flags_invalid_device_inputs_with_nan(fa):
    """A length above max_seq_len, or a block id outside the pool, makes that
    sequence's rows NaN; other sequences are unaffected and nothing faults."""
    di = W.make_decode_inputs(3, 8, 2, 128, "bf16", seed=12, seq_lens=[50, 60, 70], paged=True)
    table = di.block_table.clone()
    table[1, 2] = di.kv_capacity + 100       # bad id in a used block of sequence 1
    lens = di.seq_lens.clone()
    lens[2] = 500                            # sequence 2 claims more than max_seq_len
    o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), lens.to(DEV),
                       block_table=table.to(DEV), max_seq_len=70)
    torch.cuda.synchronize()
    o, lse = o.cpu().float(), lse.cpu()
    assert torch.isnan(o[1]).all() and torch.isnan(lse[1]).all()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()
    O_ref, lse_ref = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, 16, 128 ** -0.5,
                                         heads=[(0, h) for h in range(8)])
    check(o[0], lse[0], O_ref[0], lse_ref[0], "bf16", "good sequence")


def test_decode_writes_nothing_outside_its_output(fa):
    di = W.make_decode_inputs(3, 8, 2, 128, "bf16", seed=13, seq_lens=[900, 10, 300])
    guard = 1024
    n = 3 * 8 * 128
    buf = torch.full((n + 2 * guard,), 5.0, dtype=torch.bfloat16, device=DEV)
    out = buf[guard:guard + n].view(3, 8, 128)
    fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), split_tokens=256, out=out)
    torch.cuda.synchronize()
    assert (buf[:guard] == 5).all() and (buf[-guard:] == 5).all()


# ----------------------------------------------------------------------------
# the five workloads at full size
# ----------------------------------------------------------------------------
def test_workload_1_fp32_single_head(fa):
    w = W.C1
    q, k, v = W.prefill_inputs(w)
    O_ref, lse_ref = oracle.prefill(q, k, v, w.scale, w.causal)
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    err = check(o, lse, O_ref, lse_ref, "f32", w.name)
    note(f"{w.name}: max abs err {err:.2e}")


def _sample_rows(w, rng, n_random):
    heads = sorted({0, w.Hq - 1, w.Hq // 2, int(rng.integers(w.Hq))})
    fixed = [0, 1, 63, 64, 127, 128, 129, w.Nq // 2, w.Nq - 129, w.Nq - 128, w.Nq - 2, w.Nq - 1]
    rows = [(0, h, i) for h in heads for i in fixed]
    rows += [(0, int(rng.integers(w.Hq)), int(rng.integers(w.Nq))) for _ in range(n_random)]
    return rows


def one_head_per_kv_head(w):
    """A query head of every KV head, each at a different position within its
    group: every KV head (and with it every XCD slot of the launch's
    KV-head-major mapping), every query-tile pair, and every place a head
    takes among the query heads that share a workgroup is covered."""
    n_rep = w.Hq // w.Hkv
    return [(b, g * n_rep + (g + b) % n_rep) for b in range(w.B) for g in range(w.Hkv)]


def test_workload_prefill_full_size_C2_every_output(fa):
    """The N = 4096 workload in the benchmark's launch configuration, every
    output element and every LSE against the oracle."""
    w = W.C2
    note(f"{w.name}: generating inputs")
    q, k, v = W.prefill_inputs(w)
    note(f"{w.name}: launching")
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    note(f"{w.name}: oracle over all {w.B * w.Hq} heads")
    ref = FS.prefill_heads(q, k, v, w.scale, w.causal, [(b, h) for b in range(w.B) for h in range(w.Hq)])
    O_ref = np.stack([np.stack([ref[(b, h)][0] for h in range(w.Hq)]) for b in range(w.B)])
    L_ref = np.stack([np.stack([ref[(b, h)][1] for h in range(w.Hq)]) for b in range(w.B)])
    err = check(o_c, lse_c, O_ref, L_ref, "bf16", w.name)
    note(f"{w.name}: all {o_c.numel()} outputs, max abs err {err:.2e}")


@pytest.fixture(scope="module")
def c4_run(fa):
    w = W.C4
    note(f"{w.name}: generating inputs")
    q, k, v = W.prefill_inputs(w)
    note(f"{w.name}: launching")
    o, lse = fa.prefill(q.to(DEV), k.to(DEV), v.to(DEV), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    del o, lse
    torch.cuda.empty_cache()
    return w, q, k, v, o_c, lse_c


def test_workload_prefill_full_size_C4_whole_heads(c4_run):
    """N = 32768: every row of one query head per KV head (all 512 query-tile
    pairs of the launch, every KV head, each of the 8 places of a head in its
    workgroup) against the oracle."""
    w, q, k, v, o_c, lse_c = c4_run
    assert torch.isfinite(o_c.float()).all() and torch.isfinite(lse_c).all()
    heads = one_head_per_kv_head(w)
    note(f"{w.name}: oracle over heads {heads}")
    ref = FS.prefill_heads(q, k, v, w.scale, w.causal, heads)
    for b, h in heads:
        err = check(o_c[b, h], lse_c[b, h], ref[(b, h)][0], ref[(b, h)][1], "bf16", f"{w.name} head {h}")
        note(f"{w.name}: head {h}, all {w.Nq} rows, max abs err {err:.2e}")


def test_workload_prefill_full_size_C4_sampled_rows(c4_run):
    """N = 32768: rows sampled over all heads (tile edges and random)."""
    w, q, k, v, o_c, lse_c = c4_run
    rows = _sample_rows(w, np.random.default_rng(w.seed), 48)
    O_ref, lse_ref = oracle.prefill_rows(q, k, v, w.scale, w.causal, rows)
    got = torch.stack([o_c[b, h, i] for b, h, i in rows])
    got_lse = torch.stack([lse_c[b, h, i] for b, h, i in rows])
    err = check(got, got_lse, O_ref, lse_ref, "bf16", w.name)
    note(f"{w.name}: {len(rows)} sampled rows, max abs err {err:.2e}")


@pytest.mark.parametrize("w", [W.C3, W.C5], ids=["C3_contiguous", "C5_paged"])
def test_workload_decode_full_size_every_output(fa, w):
    """The decode workloads in the benchmark's launch configuration (library
    split choice), every (sequence, head) output and LSE against the oracle."""
    note(f"{w.name}: generating inputs")
    di = W.decode_inputs(w)
    note(f"{w.name}: launching")
    kwargs = dict(max_seq_len=di.max_seq_len)
    if di.paged:
        kwargs["block_table"] = di.block_table.to(DEV)
    o, lse = fa.decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV), **kwargs)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    note(f"{w.name}: oracle over all {w.B} sequences")
    if di.paged:
        fn = lambda heads: oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens,  # noqa: E731
                                               di.block_size, w.scale, heads=heads)
    else:
        fn = lambda heads: oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, w.scale,  # noqa: E731
                                                    heads=heads)
    O_ref, L_ref = FS.decode_batches(fn, w.B, w.Hq)
    err = check(o_c, lse_c, O_ref, L_ref, "bf16", w.name)
    note(f"{w.name}: all {w.B * w.Hq} (sequence, head) rows, max abs err {err:.2e}")
