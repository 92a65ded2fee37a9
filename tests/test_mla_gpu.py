"""MLA decode through the C ABI, against the fp64 oracle (bf16 tolerances:
max-abs 2e-2, mean-abs 2e-3 on the latent-space output; LSE 1e-4)."""
import math
import sys

import numpy as np
import pytest
import torch

import full_size as FS
import oracle
from oracle import mla as M
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1 / math.sqrt(128 + 64)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(o_gpu, lse_gpu, O_ref, lse_ref, what=""):
    O = o_gpu.detach().to("cpu", torch.float64).numpy()
    assert O.shape == np.asarray(O_ref).shape
    assert np.isfinite(O).all(), f"{what}: non-finite output"
    err = np.abs(O - O_ref)
    assert err.max() <= 2e-2, f"{what}: max abs err {err.max():.3e}"
    assert err.mean() <= 2e-3, f"{what}: mean abs err {err.mean():.3e}"
    e = np.abs(lse_gpu.detach().to("cpu", torch.float64).numpy() - lse_ref).max()
    assert e <= 1e-4, f"{what}: LSE err {e:.3e}"


CASES = [
    # B, Hq, lens, paged, block_size, split_tokens
    (2, 128, [1, 37], True, 64, 0),
    (3, 128, [32, 200, 1000], True, 64, 256),
    (3, 16, [5, 300, 2100], True, 16, 512),
    (2, 64, [129, 3000], True, 8, 1024),       # pages smaller than a wave's share of a tile
    (3, 128, [64, 65, 513], False, 0, 128),
    (2, 40, [700, 2049], True, 32, 0),         # heads not a multiple of 16
    (1, 256, [1500], True, 64, 512),           # two head groups
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_{}_bs{}_st{}".format(
    c[0], c[1], "paged" if c[3] else "contig", c[4], c[5]))
def test_mla_decode_small(fa, case):
    B, Hq, lens, paged, bs, st = case
    note(f"mla decode {case}")
    mi = W.make_mla_inputs(B, Hq, 512, 64, seed=1100 + Hq + B, seq_lens=lens, paged=paged, block_size=max(bs, 1),
                           s_cap=(max(lens) + 40) if not paged else None, spare_blocks=2 if paged else 0)
    table = mi.block_table.to(DEV) if paged else None
    o, lse = fa.mla_decode(mi.q.to(DEV), mi.kv.to(DEV), mi.seq_lens.to(DEV), SCALE, block_table=table,
                           max_seq_len=mi.max_seq_len, split_tokens=st)
    torch.cuda.synchronize()
    O_ref, lse_ref = M.mla_decode_latent(mi.q, mi.kv, mi.seq_lens, SCALE, 512,
                                         mi.block_table if paged else None, mi.block_size)
    check(o, lse, O_ref, lse_ref, f"mla {case}")


def test_mla_split_count_does_not_change_the_answer_beyond_tolerance(fa):
    mi = W.make_mla_inputs(2, 128, 512, 64, 1201, seq_lens=[3000, 4100], block_size=64)
    args = (mi.q.to(DEV), mi.kv.to(DEV), mi.seq_lens.to(DEV), SCALE)
    outs = [fa.mla_decode(*args, block_table=mi.block_table.to(DEV), max_seq_len=mi.max_seq_len, split_tokens=st)
            for st in (0, 256, 1024, 8192)]
    torch.cuda.synchronize()
    O_ref, lse_ref = M.mla_decode_latent(mi.q, mi.kv, mi.seq_lens, SCALE, 512, mi.block_table, 64)
    for o, lse in outs:
        check(o, lse, O_ref, lse_ref, "split")


def test_mla_flags_invalid_device_inputs_with_nan(fa):
    mi = W.make_mla_inputs(3, 32, 512, 64, 1202, seq_lens=[100, 100, 100], block_size=16)
    lens = mi.seq_lens.clone()
    lens[0] = mi.max_seq_len + 1
    table = mi.block_table.clone()
    table[1, 3] = mi.kv_capacity + 1
    o, lse = fa.mla_decode(mi.q.to(DEV), mi.kv.to(DEV), lens.to(DEV), SCALE, block_table=table.to(DEV),
                           max_seq_len=mi.max_seq_len)
    torch.cuda.synchronize()
    o, lse = o.float().cpu(), lse.cpu()
    assert torch.isnan(o[:2]).all() and torch.isnan(lse[:2]).all()
    O_ref, lse_ref = M.mla_decode_latent(mi.q[2:], mi.kv, mi.seq_lens[2:], SCALE, 512, mi.block_table[2:], 16)
    check(o[2:], lse[2:], O_ref, lse_ref, "valid sequence next to invalid ones")


def test_mla_kernel_implements_the_absorbed_model(fa):
    """Through the kernel, then W^UV: the explicit per-head MLA of the page's
    equations (reconstructed keys and values, decoupled position key)."""
    B, H, d_head, S = 2, 16, 128, 300
    g = torch.Generator().manual_seed(1203)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    q_c, q_r = r(B, H, d_head), r(B, H, 64)
    w_uk, w_uv = r(H, d_head, 512) / math.sqrt(512), r(H, d_head, 512) / math.sqrt(512)
    latent, k_rope = r(B, S, 512), r(B, S, 64)
    lens = torch.tensor([S, 123], dtype=torch.int32)
    q = torch.cat([torch.tensor(M.absorb_query(q_c, w_uk)), q_r], dim=2).to(torch.bfloat16)
    kv = torch.cat([latent, k_rope], dim=2).to(torch.bfloat16)
    o, lse = fa.mla_decode(q.to(DEV), kv.to(DEV), lens.to(DEV), SCALE)
    torch.cuda.synchronize()
    # the explicit per-head model, in fp64 on the unrounded inputs
    Oe, le = M.mla_decode_explicit(q_c, q_r, w_uk, w_uv, latent, k_rope, lens, SCALE)
    head = M.latent_to_head(o.double().cpu().numpy(), w_uv)
    assert np.abs(head - Oe).max() < 2e-2
    assert np.abs(lse.double().cpu().numpy() - le).max() < 2e-2   # bf16 rounding of q and the cache


def test_mla_decode_full_size(fa):
    """The DeepSeek-V3-shaped MLA batch in the benchmark's launch
    configuration: every (sequence, head) output and LSE against the oracle."""
    w = W.MLA_DECODE
    note(f"mla decode {w.name}")
    mi = W.mla_inputs(w)
    o, lse = fa.mla_decode(mi.q.to(DEV), mi.kv.to(DEV), mi.seq_lens.to(DEV), w.scale,
                           block_table=mi.block_table.to(DEV), max_seq_len=mi.max_seq_len)
    torch.cuda.synchronize()
    note("mla decode: oracle over the whole batch")
    O_ref, lse_ref = FS.decode_batches(
        lambda heads: M.mla_decode_latent(mi.q, mi.kv, mi.seq_lens, w.scale, 512, mi.block_table, w.block_size,
                                          heads=heads), w.B, w.Hq)
    check(o.cpu(), lse.cpu(), O_ref, lse_ref, "mla full size, every output")


def _expected_items(lens, max_seq_len, st):
    """(item id, tile count) of every split the work list must hold: a valid
    length L gives ceil(L / st) parts of equal length rounded up to 32 tokens,
    an invalid one a single (NaN-flagging) item; ids are b * max_splits + s."""
    ns_max = 1 if max_seq_len <= st else -(-max_seq_len // st)
    items = {}
    for b, L in enumerate(lens):
        bad = L < 0 or L > max_seq_len
        ns = 1 if bad else max(1, -(-L // st))
        sl = L if ns <= 1 else -(-(-(-L // ns)) // 32) * 32
        for s in range(ns):
            t0 = s * sl
            t1 = min(L, t0 + sl)
            items[b * ns_max + s] = 0 if bad else min(1023, -(-(t1 - t0) // 32))
    return items, ns_max


@pytest.mark.parametrize("st", [4096, 24576])
def test_mla_work_list_orders_every_split_longest_first(fa, st):
    # Many sequences over a tiny pool (block ids repeat), so that lengths up to
    # 40000 tokens cost little memory and the tile counts spread over most of
    # the sort's buckets.
    B, Hq, bs, nblk, max_len = 300, 16, 64, 32, 40000
    g = torch.Generator().manual_seed(1300 + st)
    lens = torch.randint(0, max_len + 1, (B,), generator=g, dtype=torch.int32)
    lens[:4] = torch.tensor([0, 1, max_len, -1], dtype=torch.int32)
    max_blocks = -(-max_len // bs)
    table = torch.randint(0, nblk, (B, max_blocks), generator=g, dtype=torch.int32)
    q = torch.randn((B, Hq, 576), generator=g).to(torch.bfloat16)
    kv = torch.randn((nblk, bs, 576), generator=g).to(torch.bfloat16)
    note(f"mla work list B={B} st={st}")
    need = fa.mla_decode_workspace_bytes(B, Hq, max_len, st)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o, lse = fa.mla_decode(q.to(DEV), kv.to(DEV), lens.to(DEV), SCALE, block_table=table.to(DEV), max_seq_len=max_len,
                           split_tokens=st, workspace=ws)
    torch.cuda.synchronize()
    items, ns = _expected_items(lens.tolist(), max_len, st)
    slots = B * Hq * ns
    # workspace: bf16 partial outputs, fp32 partial LSEs, then the plan (each 256-byte aligned)
    off = -(-slots * 512 * 2 // 256) * 256 + -(-slots * 4 // 256) * 256
    plan = ws[off:off + 4 * (1 + len(items))].cpu().view(torch.int32).tolist()
    assert plan[0] == len(items)
    order = plan[1:]
    assert sorted(order) == sorted(items)
    tiles = [items[i] for i in order]
    assert all(x >= y for x, y in zip(tiles, tiles[1:])), "work list not longest first"
    lse_h = lse.cpu()
    assert torch.isnan(lse_h[3]).all() and torch.isfinite(lse_h[4:]).all()
    # two sampled sequences against the oracle (paged reads through the repeated block ids)
    for b in (2, 5):
        L = int(lens[b])
        O_ref, lse_ref = M.mla_decode_latent(q[b:b + 1], kv, lens[b:b + 1], SCALE, 512, table[b:b + 1], bs)
        check(o[b:b + 1], lse[b:b + 1], O_ref, lse_ref, f"work list seq {b} L={L}")
