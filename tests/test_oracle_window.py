"""Pins of the sliding-window reading of the oracle (CPU only).

The page prints the window-3 mask over six positions; the rest follows from
the definition: a window at least as long as the sequence is plain causal
attention, a window of one key returns the query's own value, and a windowed
row is plain attention over the slice of keys it sees.  The last test plants
an off-by-one in the window and shows that the printed mask catches it.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from flashattention_kv_cache_amd.workloads import make_chunked_inputs, make_decode_inputs, make_prefill_inputs

from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def visible(Nq, Nk, window):
    """The (Nq, Nk) 0/1 matrix of keys the oracle lets each query see."""
    m = np.zeros((Nq, Nk), dtype=int)
    for i in range(Nq):
        m[i, A.window_key_start(i, Nq, Nk, window):A.causal_key_limit(i, Nq, Nk)] = 1
    return m


def test_printed_window_mask():
    g = golden("sliding_window_mask.json")
    assert visible(g["n"], g["n"], g["window"]).tolist() == g["mask"]


def test_printed_mask_through_attention():
    """Scores that make each visible key's weight observable: with V = I, row i
    of O is the softmax row, so its support is the mask row."""
    g = golden("sliding_window_mask.json")
    n = g["n"]
    q = torch.zeros(1, 1, n, 4, dtype=torch.float64)
    k = torch.zeros(1, 1, n, 4, dtype=torch.float64)
    v = torch.eye(n, dtype=torch.float64)[None, None]
    O, _ = oracle.prefill(q, k, v, 1.0, True, window=g["window"])
    assert ((O[0, 0] > 0).astype(int)).tolist() == g["mask"]
    np.testing.assert_allclose(O[0, 0].sum(axis=1), 1.0, atol=1e-15)


@pytest.mark.parametrize("Nq,Nk", [(7, 7), (3, 10)])
def test_window_at_least_the_sequence_is_causal(Nq, Nk):
    q, k, v = make_prefill_inputs(1, 4, 2, Nq, Nk, 16, "f32", seed=3)
    O, lse = oracle.prefill(q, k, v, 0.25, True)
    for W in (Nk, Nk + 5):
        Ow, lw = oracle.prefill(q, k, v, 0.25, True, window=W)
        assert np.array_equal(O, Ow) and np.array_equal(lse, lw)


def test_window_of_one_key_is_the_own_value():
    q, k, v = make_prefill_inputs(1, 2, 1, 5, 9, 8, "f32", seed=4)
    O, lse = oracle.prefill(q, k, v, 0.5, True, window=1)
    for i in range(5):
        p = i + 4                               # bottom-right: query i is position i + Nk - Nq
        np.testing.assert_allclose(O[0, :, i], np.broadcast_to(v[0, 0, p].double().numpy(), (2, 8)), atol=1e-15)
        s = 0.5 * (q[0, :, i].double() @ k[0, 0, p].double()).numpy()
        np.testing.assert_allclose(lse[0, :, i], s, atol=1e-14)


def test_windowed_row_is_plain_attention_over_its_slice():
    q, k, v = make_prefill_inputs(1, 2, 1, 12, 20, 8, "f32", seed=5)
    W = 5
    O, lse = oracle.prefill(q, k, v, 0.3, True, window=W)
    for i in (0, 4, 11):
        p = i + 8
        lo = max(0, p - W + 1)
        Ks, Vs = k[0, 0, lo:p + 1].double().numpy(), v[0, 0, lo:p + 1].double().numpy()
        for h in range(2):
            s = 0.3 * Ks @ q[0, h, i].double().numpy()
            w = np.exp(s - s.max())
            np.testing.assert_allclose(O[0, h, i], (w / w.sum()) @ Vs, atol=1e-14)
            np.testing.assert_allclose(lse[0, h, i], s.max() + np.log(w.sum()), atol=1e-14)
    Or, lr = oracle.prefill_rows(q, k, v, 0.3, True, [(0, 1, 4), (0, 0, 11)], window=W)
    np.testing.assert_allclose(Or, np.stack([O[0, 1, 4], O[0, 0, 11]]), atol=1e-14)


def test_windowed_decode_is_decode_over_the_last_keys():
    di = make_decode_inputs(3, 4, 2, 16, "bf16", 6, seq_lens=[3, 20, 41], paged=True, block_size=4)
    W = 8
    O, lse = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, 4, 0.25, window=W)
    for b, L in enumerate(di.seq_lens.tolist()):
        lo = max(0, L - W)
        for h in range(4):
            K = A.paged_gather(di.k_cache, di.block_table[b], L, h // 2, 4)[lo:]
            V = A.paged_gather(di.v_cache, di.block_table[b], L, h // 2, 4)[lo:]
            o, l = A.attention_rows(di.q[b, h:h + 1], K, V, 0.25)
            np.testing.assert_allclose(O[b, h], o[0], atol=1e-14)
            np.testing.assert_allclose(lse[b, h], l[0], atol=1e-14)
    # contiguous agrees with paged
    cap = 41
    kc = torch.full((3, 2, cap, 16), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    for b, L in enumerate(di.seq_lens.tolist()):
        for j in range(L):
            kc[b, :, j] = di.k_cache[int(di.block_table[b, j // 4]), j % 4]
            vc[b, :, j] = di.v_cache[int(di.block_table[b, j // 4]), j % 4]
    Oc, lc = oracle.decode_contiguous(di.q, kc, vc, di.seq_lens, 0.25, window=W)
    np.testing.assert_allclose(Oc, O, atol=1e-14)


def test_windowed_chunk_is_rows_of_windowed_prefill():
    ci = make_chunked_inputs(2, 4, 2, 16, "f32", 7, chunk=5, past_lens=[9, 2], block_size=4)
    kr, vr = oracle.append_batch(ci.k_cache, ci.v_cache, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 4)
    W = 6
    O, lse = oracle.chunked_prefill(ci.q, kr, vr, ci.seq_lens, 0.3, True, ci.block_table, 4, window=W)
    for b in range(2):
        L = int(ci.seq_lens[b])
        K = torch.stack([torch.tensor(A.paged_gather(kr, ci.block_table[b], L, g, 4)) for g in range(2)])[None]
        V = torch.stack([torch.tensor(A.paged_gather(vr, ci.block_table[b], L, g, 4)) for g in range(2)])[None]
        Of, lf = oracle.prefill(ci.q[b:b + 1], K, V, 0.3, True, window=W)
        np.testing.assert_allclose(O[b], Of[0], atol=1e-14)
        np.testing.assert_allclose(lse[b], lf[0], atol=1e-14)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(A, "window_key_start", lambda i, Nq, Nk, w: 0 if w <= 0 else max(0, i + Nk - Nq - w))
    with pytest.raises(AssertionError):
        test_printed_window_mask()
