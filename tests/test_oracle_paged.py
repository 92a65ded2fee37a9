"""Pins of the paged-cache oracle: block allocation, append, prefix sharing and
chunked prefill (CPU only).

The printed outputs of the paging demos (tests/golden/paging_demo.json) fix
the allocator and the slot rule; bit-exact gathers fix the append; the rows of
the already pinned full causal prefill and decode fix the chunked prefill.  The
last tests plant mistakes in the oracle and show that a pin catches each.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import paged as PG
from flashattention_kv_cache_amd.workloads import make_chunked_inputs

from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _gather_tokens(pool, table_row, L, bs):
    """(L, H_kv, d) of one sequence, read slot by slot through its table."""
    return torch.stack([pool[int(table_row[t // bs]), t % bs] for t in range(L)]) if L else pool[:0, 0]


# --------------------------------------------------------------------------
# the demos the page prints
# --------------------------------------------------------------------------
def test_tiny_demo_table_and_gather():
    t = golden("paging_demo.json")["tiny"]
    pk = torch.zeros(t["num_blocks"], t["block_size"], t["num_kv_heads"], t["head_dim"])
    pv = pk.clone()
    alloc = PG.BlockAllocator(t["num_blocks"])
    seq = PG.PagedSequence()
    g = torch.Generator().manual_seed(0)
    toks = [(torch.randn(t["num_kv_heads"], t["head_dim"], generator=g),
             torch.randn(t["num_kv_heads"], t["head_dim"], generator=g)) for _ in range(t["tokens"])]
    for k, v in toks:
        PG.append_token(pk, pv, alloc, seq, k, v)
    assert seq.length == t["tokens"]
    assert len(seq.table) == t["blocks_used"] == alloc.num_used
    assert seq.table == t["block_table"]
    assert alloc.num_free + alloc.num_used == t["num_blocks"]
    gk = _gather_tokens(pk, seq.table, seq.length, t["block_size"])
    assert list(gk.shape) == t["gathered_shape"]
    assert torch.equal(gk, torch.stack([k for k, _ in toks])) == t["paged_equals_contiguous"]
    # the attention-side reader agrees with the slot-by-slot gather
    for h in range(t["num_kv_heads"]):
        assert np.array_equal(A.paged_gather(pv, seq.table, seq.length, h, t["block_size"]),
                              torch.stack([v for _, v in toks])[:, h].double().numpy())


def test_serving_demo_blocks_and_gather():
    s = golden("paging_demo.json")["serving"]
    bs = s["block_size"]
    nb = s["contiguous_slots"] // bs
    pk = torch.zeros(nb, bs, 1, 4)
    pv = pk.clone()
    alloc = PG.BlockAllocator(nb)
    g = torch.Generator().manual_seed(1)
    ok = True
    seqs = []
    for L in s["lengths"]:
        seq = PG.PagedSequence()
        ks = torch.randn(L, 1, 4, generator=g)
        for i in range(L):
            PG.append_token(pk, pv, alloc, seq, ks[i], -ks[i])
        ok &= torch.equal(_gather_tokens(pk, seq.table, L, bs), ks)
        seqs.append(seq)
    assert ok == s["gather_equals_contiguous"]
    assert alloc.num_used == s["paged_blocks"]
    assert alloc.num_used * bs == s["paged_slots"]
    assert alloc.num_used * bs - sum(s["lengths"]) == s["paged_waste_tokens"]
    # freeing gives every block back
    for seq in seqs:
        for blk in seq.table:
            alloc.release(blk)
    assert alloc.num_used == 0
    with pytest.raises(ValueError):
        alloc.release(0)


def test_sharing_demo():
    s = golden("paging_demo.json")["sharing"]
    pk = torch.zeros(s["num_blocks"], s["block_size"], s["num_kv_heads"], s["head_dim"])
    pv = pk.clone()
    alloc = PG.BlockAllocator(s["num_blocks"])
    prompt = PG.PagedSequence()
    for _ in range(s["prompt_tokens"]):
        PG.append_token(pk, pv, alloc, prompt, torch.ones(1, 2), torch.ones(1, 2))
    assert alloc.num_used == s["blocks_used_before"]
    sample = PG.share_prefix(prompt, s["shared_prefix_blocks"])
    assert alloc.num_used == s["blocks_used_after"]
    assert (sample.table[0] == prompt.table[0]) == s["same_physical_prefix_block"]
    with pytest.raises(ValueError):
        PG.share_prefix(prompt, 3)


# --------------------------------------------------------------------------
# batched append: bit-exact placement
# --------------------------------------------------------------------------
@pytest.mark.parametrize("paged,bs", [(True, 16), (True, 4), (True, 1), (False, 0)])
def test_append_batch_is_the_concatenation(paged, bs):
    ci = make_chunked_inputs(3, 4, 2, 8, "bf16", 11, chunk=9, past_lens=[0, 23, 16], paged=paged,
                             block_size=max(bs, 1), spare_blocks=2)
    n = ci.k_new.shape[2]
    if paged:
        k2, v2 = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, bs)
    else:
        k2, v2 = oracle.append_batch_contiguous(ci.k_cache, ci.v_cache, ci.seq_lens, ci.k_new, ci.v_new)
    written = torch.zeros(k2.shape[:-1], dtype=torch.bool)
    for b in range(3):
        L = int(ci.seq_lens[b])
        for g in range(2):
            if paged:
                before = _gather_tokens(ci.k_cache, ci.block_table[b], L - n, bs)[:, g] if L > n else None
                after = _gather_tokens(k2, ci.block_table[b], L, bs)[:, g]
                after_v = _gather_tokens(v2, ci.block_table[b], L, bs)[:, g]
            else:
                before = ci.k_cache[b, g, :L - n]
                after, after_v = k2[b, g, :L], v2[b, g, :L]
            if before is not None:
                assert torch.equal(after[:L - n], before)
            assert torch.equal(after[L - n:], ci.k_new[b, g]) and torch.equal(after_v[L - n:], ci.v_new[b, g])
            assert not torch.isnan(after).any()
        for t in range(L - n, L):
            if paged:
                written[int(ci.block_table[b, t // bs]), t % bs] = True
            else:
                written[b, :, t] = True
    # every slot the append does not own is untouched (NaN poison included)
    same = torch.isclose(k2, ci.k_cache, equal_nan=True).all(-1)
    assert same[~written].all()


# --------------------------------------------------------------------------
# chunked prefill = rows of the pinned full causal prefill / decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("paged", [True, False])
def test_chunked_prefill_equals_last_rows_of_full_causal(paged):
    B, Hq, Hkv, d, n = 2, 4, 2, 16, 6
    ci = make_chunked_inputs(B, Hq, Hkv, d, "bf16", 12, chunk=n, past_lens=[13, 4], paged=paged, block_size=4)
    if paged:
        k2, v2 = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 4)
    else:
        k2, v2 = oracle.append_batch_contiguous(ci.k_cache, ci.v_cache, ci.seq_lens, ci.k_new, ci.v_new)
    O, lse = oracle.chunked_prefill(ci.q, k2, v2, ci.seq_lens, 0.3, True, ci.block_table, ci.block_size)
    for b in range(B):
        L = int(ci.seq_lens[b])
        K = torch.stack([torch.tensor(A.paged_gather(k2, ci.block_table[b], L, g, 4)) if paged
                         else k2[b, g, :L].double() for g in range(Hkv)])[None]
        V = torch.stack([torch.tensor(A.paged_gather(v2, ci.block_table[b], L, g, 4)) if paged
                         else v2[b, g, :L].double() for g in range(Hkv)])[None]
        # full causal prefill over L tokens whose last n queries are ours
        qf = torch.randn(1, Hq, L, d, dtype=torch.float64)
        qf[:, :, L - n:] = ci.q[b:b + 1].double()
        Of, lf = oracle.prefill(qf, K, V, 0.3, True)
        np.testing.assert_allclose(O[b], Of[0, :, L - n:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], lf[0, :, L - n:], rtol=0, atol=1e-13)
        # and it is the (bottom-right) causal prefill of the chunk against its cache
        Oc, lc = oracle.prefill(ci.q[b:b + 1], K, V, 0.3, True)
        np.testing.assert_allclose(O[b], Oc[0], rtol=0, atol=1e-13)
    # selected rows agree with the whole computation
    rows = [(0, 3, 0), (1, 1, 5), (1, 0, 2)]
    Or, lr = oracle.chunked_prefill(ci.q, k2, v2, ci.seq_lens, 0.3, True, ci.block_table, ci.block_size, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(Or[r], O[b, h, i], rtol=0, atol=1e-13)
        assert abs(lr[r] - lse[b, h, i]) < 1e-13


def test_chunked_prefill_of_one_token_is_decode():
    ci = make_chunked_inputs(3, 4, 1, 8, "f32", 13, chunk=1, past_lens=[0, 7, 30], block_size=8)
    k2, v2 = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 8)
    O, lse = oracle.chunked_prefill(ci.q, k2, v2, ci.seq_lens, 0.5, True, ci.block_table, 8)
    Od, ld = oracle.decode_paged(ci.q[:, :, 0], k2, v2, ci.block_table, ci.seq_lens, 8, 0.5)
    np.testing.assert_allclose(O[:, :, 0], Od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[:, :, 0], ld, rtol=0, atol=1e-13)


def test_chunked_prefill_non_causal_sees_whole_cache():
    ci = make_chunked_inputs(1, 2, 1, 8, "f32", 14, chunk=3, past_lens=[5], block_size=2)
    k2, v2 = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 2)
    O, lse = oracle.chunked_prefill(ci.q, k2, v2, ci.seq_lens, 0.5, False, ci.block_table, 2)
    Od0, _ = oracle.decode_paged(ci.q[:, :, 0], k2, v2, ci.block_table, ci.seq_lens, 2, 0.5)
    np.testing.assert_allclose(O[:, :, 0], Od0, rtol=0, atol=1e-13)   # every row sees all 8 keys


def test_shared_prefix_blocks_are_read_by_both():
    ci = make_chunked_inputs(2, 2, 1, 8, "f32", 15, chunk=2, past_lens=[9, 12], block_size=4,
                             shared_prefix_blocks=2)
    assert torch.equal(ci.block_table[0, :2], ci.block_table[1, :2])
    k2, v2 = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 4)
    a = A.paged_gather(k2, ci.block_table[0], 8, 0, 4)
    b = A.paged_gather(k2, ci.block_table[1], 8, 0, 4)
    assert np.array_equal(a, b) and not np.isnan(a).any()


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def test_planted_append_slot_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(PG, "slot_of", lambda row, t, bs: (int(row[t // bs]), (t + 1) % bs))
    with pytest.raises(AssertionError):
        test_append_batch_is_the_concatenation(True, 4)


def test_planted_append_position_is_caught(monkeypatch):
    real = PG.slot_of
    monkeypatch.setattr(PG, "slot_of", lambda row, t, bs: real(row, t + 1, bs))
    with pytest.raises((AssertionError, IndexError, ValueError)):
        test_append_batch_is_the_concatenation(True, 16)


def test_planted_top_left_chunk_mask_is_caught(monkeypatch):
    real = A.attention_rows

    def top_left(q_rows, K, V, scale, key_limits=None, key_starts=None):
        if key_limits is not None and len(key_limits) > 1:
            key_limits = [i + 1 for i in range(len(key_limits))]
        return real(q_rows, K, V, scale, key_limits, key_starts)

    monkeypatch.setattr(PG, "attention_rows", top_left)
    with pytest.raises(AssertionError):
        test_chunked_prefill_equals_last_rows_of_full_causal(True)
