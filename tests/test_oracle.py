"""Pins of the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/*.json, each with its citation), closed forms,
special cases that reduce to a library routine, pure-Python brute force on tiny
inputs, and a second algorithm (the pages' streaming recurrence).  The last
group plants plausible mistakes in a copy of the oracle and shows that a pin
catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import online as OL
from flashattention_kv_cache_amd.workloads import make_decode_inputs, make_prefill_inputs

from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# P1: the worked example of the running max / running sum recurrence
# --------------------------------------------------------------------------
def test_p1_worked_example_recurrence():
    g = golden("online_softmax_worked_example.json")
    stats = OL.online_softmax_stats(g["scores"], g["block"])
    tol = 0.5 * 10 ** -g["printed_decimals"]
    for (d_k, s_k), want in zip(stats, g["after_block"]):
        assert d_k == want["d"]
        assert abs(s_k - want["s"]) <= tol
    terms = [math.exp(a - 4) for a in g["scores"]]
    for t, want in zip(terms, g["direct_terms"]):
        assert abs(t - want) <= tol
    assert abs(stats[-1][1] - g["direct_sum"]) <= tol


def test_p1_worked_example_pins_oracle_lse():
    """The oracle's LSE of the example's scores is d_2 + ln s_2."""
    g = golden("online_softmax_worked_example.json")
    K = np.array(g["scores"], dtype=np.float64)[:, None]
    V = np.eye(4)
    O, lse = A.attention_rows(np.ones((1, 1)), K, V, scale=1.0)
    want_lse = g["after_block"][-1]["d"] + math.log(g["after_block"][-1]["s"])
    assert abs(lse[0] - want_lse) < 1e-3
    # with V = I the output row is the softmax itself: e^{a_i - 4} / s_2
    want_p = np.array(g["direct_terms"]) / g["direct_sum"]
    assert np.allclose(O[0], want_p, atol=2e-3)


# --------------------------------------------------------------------------
# P2: streaming (online) softmax equals the two-pass definition
# --------------------------------------------------------------------------
@pytest.mark.parametrize("block", [1, 4, 7, 64])
def test_p2_online_equals_two_pass_fp64(block):
    r = rng(1)
    N, d = 37, 16
    q = r.normal(size=d)
    K = r.normal(size=(N, d))
    V = r.normal(size=(N, d))
    scale = 1 / math.sqrt(d)
    O_ref, lse_ref = A.attention_rows(q[None], K, V, scale)
    O_on, lse_on = OL.online_attention_row(q, K, V, scale, block)
    # the lecture notes expect about 1e-15 in float64
    assert np.max(np.abs(O_on - O_ref[0])) < 1e-14
    assert abs(lse_on - lse_ref[0]) < 1e-13


def test_p2_notebook_fp32_streaming_within_1e5():
    """Shape and tolerance of the notebook's online-softmax check: (2,4,12,16),
    key blocks of 4, fp32 streaming vs the definition within 1e-5."""
    torch.manual_seed(0)
    q = torch.randn(2, 4, 12, 16)
    k = torch.randn(2, 4, 12, 16)
    v = torch.randn(2, 4, 12, 16)
    O_ref, _ = A.prefill(q, k, v, 16 ** -0.5, causal=False)
    # fp32 streaming in the pages' unnormalised-accumulator form
    qn, kn, vn = q.numpy(), k.numpy(), v.numpy()
    worst = 0.0
    for b in range(2):
        for h in range(4):
            for i in range(12):
                m = np.float32(-np.inf)
                s = np.float32(0)
                acc = np.zeros(16, np.float32)
                for st in range(0, 12, 4):
                    sc = (kn[b, h, st:st + 4] @ qn[b, h, i]) * np.float32(0.25)
                    new_m = max(m, sc.max())
                    old = np.float32(0) if m == -np.inf else np.exp(m - new_m)
                    e = np.exp(sc - new_m)
                    s = s * old + e.sum()
                    acc = acc * old + e @ vn[b, h, st:st + 4]
                    m = new_m
                worst = max(worst, float(np.abs(acc / s - O_ref[b, h, i]).max()))
    assert worst < 1e-5


# --------------------------------------------------------------------------
# P3: decoding through the cache equals the matching row of a full causal pass
# --------------------------------------------------------------------------
def test_p3_step_by_step_decode_equals_full_causal():
    """The pages' main test of any cache: decode one token at a time, appending
    its k, v, and compare with one causal pass over the whole sequence."""
    r = rng(3)
    Hq, Hkv, N, d = 4, 2, 9, 8
    q = r.normal(size=(1, Hq, N, d))
    k = r.normal(size=(1, Hkv, N, d))
    v = r.normal(size=(1, Hkv, N, d))
    O_full, lse_full = A.prefill(q, k, v, 0.3, causal=True)
    for t in range(N):
        O_t, lse_t = A.decode_contiguous(q[:, :, t], k, v, np.array([t + 1]), 0.3)
        assert np.allclose(O_t[0], O_full[0, :, t], atol=1e-13, rtol=0)
        assert np.allclose(lse_t[0], lse_full[0, :, t], atol=1e-13, rtol=0)


def test_p3_chunked_prefill_rows_equal_full_causal():
    """A chunk of N_q queries appended to a cache of N_k - N_q keys (bottom-right
    mask) equals the last N_q rows of the full causal pass."""
    r = rng(4)
    N, Nq, d = 11, 4, 8
    q = r.normal(size=(1, 2, N, d))
    k = r.normal(size=(1, 1, N, d))
    v = r.normal(size=(1, 1, N, d))
    O_full, lse_full = A.prefill(q, k, v, 0.5, causal=True)
    O_c, lse_c = A.prefill(q[:, :, N - Nq:], k, v, 0.5, causal=True)
    assert np.allclose(O_c, O_full[:, :, N - Nq:], atol=1e-13)
    assert np.allclose(lse_c, lse_full[:, :, N - Nq:], atol=1e-13)


# --------------------------------------------------------------------------
# P4: grouped-query heads
# --------------------------------------------------------------------------
def test_p4_gqa_equals_mha_on_repeat_interleaved_kv():
    r = rng(5)
    B, Hq, Hkv, N, d = 2, 8, 2, 7, 8
    q = r.normal(size=(B, Hq, N, d))
    k = r.normal(size=(B, Hkv, N, d))
    v = r.normal(size=(B, Hkv, N, d))
    O_g, lse_g = A.prefill(q, k, v, 0.35, causal=True)
    k_rep = np.repeat(k, Hq // Hkv, axis=1)        # repeat_interleave on the head axis
    v_rep = np.repeat(v, Hq // Hkv, axis=1)
    O_m, lse_m = A.prefill(q, k_rep, v_rep, 0.35, causal=True)
    assert np.array_equal(O_g, O_m) and np.array_equal(lse_g, lse_m)
    # the tile mapping (head h -> h % Hkv) gives a different answer
    k_tile = np.tile(k, (1, Hq // Hkv, 1, 1))
    v_tile = np.tile(v, (1, Hq // Hkv, 1, 1))
    O_t, _ = A.prefill(q, k_tile, v_tile, 0.35, causal=True)
    assert not np.allclose(O_t, O_g)


def test_p4_mapping_and_divisibility():
    assert [A.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    assert [A.kv_head_of(h, 8, 1) for h in range(8)] == [0] * 8
    with pytest.raises(ValueError):
        A.kv_head_of(0, 8, 3)


# --------------------------------------------------------------------------
# P5: paged reads equal contiguous reads
# --------------------------------------------------------------------------
def test_p5_paged_gather_is_bit_equal_to_contiguous():
    g = golden("paging_demo.json")
    t = g["tiny"]
    assert (t["tokens"] + t["block_size"] - 1) // t["block_size"] == t["blocks_used"]
    di = make_decode_inputs(3, 4, 2, 8, "bf16", 7, seq_lens=[5, 33, 16], paged=True,
                            block_size=4, spare_blocks=3)
    for b in range(3):
        L = int(di.seq_lens[b])
        for gh in range(2):
            got = A.paged_gather(di.k_cache, di.block_table[b], L, gh, 4)
            want = np.stack([A._f64(di.k_cache[int(di.block_table[b, j // 4]), j % 4, gh]) for j in range(L)])
            assert np.array_equal(got, want) and not np.isnan(got).any()


def test_p5_paged_decode_equals_contiguous_decode():
    di = make_decode_inputs(3, 4, 2, 16, "bf16", 8, seq_lens=[5, 33, 16], paged=True, block_size=4)
    B, Hq, Hkv, d = 3, 4, 2, 16
    cap = 40
    kc = torch.full((B, Hkv, cap, d), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    for b in range(B):
        L = int(di.seq_lens[b])
        for j in range(L):
            kc[b, :, j] = di.k_cache[int(di.block_table[b, j // 4]), j % 4]
            vc[b, :, j] = di.v_cache[int(di.block_table[b, j // 4]), j % 4]
    O_p, lse_p = A.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, 4, 0.25)
    O_c, lse_c = A.decode_contiguous(di.q, kc, vc, di.seq_lens, 0.25)
    assert np.array_equal(O_p, O_c) and np.array_equal(lse_p, lse_c)


def test_p5_paging_demo_block_counts():
    s = golden("paging_demo.json")["serving"]
    bs = s["block_size"]
    blocks = sum((L + bs - 1) // bs for L in s["lengths"])
    assert blocks == s["paged_blocks"]
    assert blocks * bs == s["paged_slots"]
    assert len(s["lengths"]) * s["contiguous_reserve_per_seq"] == s["contiguous_slots"]
    assert round(100 * (1 - s["paged_slots"] / s["contiguous_slots"]), 1) == s["waste_percent"]
    assert s["paged_slots"] - sum(s["lengths"]) == s["paged_waste_tokens"]
    assert int(s["contiguous_slots"] / sum(s["lengths"])) == s["reserve_ratio_x"]
    # the seeded generator hands out exactly that many blocks
    di = make_decode_inputs(4, 1, 1, 8, "bf16", 0, seq_lens=s["lengths"], paged=True, block_size=bs)
    assert di.kv_capacity == s["paged_blocks"]
    assert sorted(int(x) for x in di.block_table.flatten() if x >= 0) == list(range(blocks))


# --------------------------------------------------------------------------
# P6: the KV-cache byte formula
# --------------------------------------------------------------------------
def test_p6_kv_bytes_exact():
    for e in golden("kv_cache_sizes.json")["exact_bytes"]:
        got = oracle.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["tokens"],
                                    e["batch"], e["bytes_per_elem"])
        assert got == e["bytes"], e["what"]


def test_p6_kv_bytes_table():
    unit = {"KiB": 2 ** 10, "MiB": 2 ** 20, "GiB": 2 ** 30}
    for e in golden("kv_cache_sizes.json")["binary_units"]:
        got = oracle.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["tokens"], e["batch"], 2)
        assert got == e["value"] * unit[e["unit"]], e["what"]


def _pin_bytes_per_token(fn):
    """Per-token figures the pages print: per token per layer (layers = 1),
    per head (kv_heads = 1) and per token over all layers."""
    for e in golden("kv_cache_sizes.json")["exact_bytes"]:
        if e["tokens"] == 1 and e["batch"] == 1:
            assert fn(e["layers"], e["kv_heads"], e["head_dim"], e["bytes_per_elem"]) == e["bytes"], e["what"]
    unit = {"KiB": 2 ** 10, "MiB": 2 ** 20, "GiB": 2 ** 30}
    for e in golden("kv_cache_sizes.json")["binary_units"]:
        if e["tokens"] == 1 and e["batch"] == 1:
            assert fn(e["layers"], e["kv_heads"], e["head_dim"], 2) == e["value"] * unit[e["unit"]], e["what"]
    # Llama 3 70B ("KV Cache, Flash Attention and Inference Optimization", KV
    # cache sizing): 4,096 B per token per layer in fp16, so 80 layers x 32,000
    # tokens is the printed ~10.4 GB (10.49e9 B)
    assert fn(1, 8, 128, 2) == 4096
    assert abs(fn(80, 8, 128, 2) * 32000 / 1e9 - 10.4) < 0.1
    # "Генерация и KV-кэш", "Сколько весит KV-кэш": 2 bytes per number in
    # BF16, 1 in FP8, so an FP8 cache is half the size
    assert fn(1, 8, 128, 1) * 2 == fn(1, 8, 128, 2)


def test_p6_kv_bytes_per_token():
    _pin_bytes_per_token(oracle.kv_bytes_per_token)


@pytest.mark.parametrize("kind", ["no_kv_factor", "ignores_dtype", "query_heads"])
def test_p6_planted_per_token_mistakes_are_caught(kind):
    def mutant(layers, kv_heads, head_dim, bytes_per_elem=2):
        if kind == "no_kv_factor":
            return layers * kv_heads * head_dim * bytes_per_elem
        if kind == "ignores_dtype":
            return 2 * layers * kv_heads * head_dim * 2
        return 2 * layers * (4 * kv_heads) * head_dim * bytes_per_elem  # counts query heads (n_rep = 4)
    with pytest.raises(AssertionError):
        _pin_bytes_per_token(mutant)


def test_p6_decode_workload_bytes_per_token():
    """The benchmark's byte count of a cached token equals the formula."""
    from flashattention_kv_cache_amd import workloads as W
    for w in (W.C3, W.C5, W.WINDOW_DECODE):
        assert w.kv_bytes_per_token() == oracle.kv_bytes_per_token(1, w.Hkv, w.d, 2) == 4096
    assert W.FP8_DECODE.kv_bytes_per_token() == oracle.kv_bytes_per_token(1, 8, 128, 1) == 2048


def test_p6_decode_workload_kv_bytes_match_formula():
    di = make_decode_inputs(5, 8, 2, 64, "bf16", 9, len_range=(3, 40))
    total = int(di.seq_lens.sum())
    assert di.kv_bytes() == oracle.kv_cache_bytes(1, 2, 64, total, 1, 2)


# --------------------------------------------------------------------------
# P7: special cases with closed forms
# --------------------------------------------------------------------------
def test_p7_single_key():
    r = rng(6)
    q, K, V = r.normal(size=(3, 8)), r.normal(size=(1, 8)), r.normal(size=(1, 8))
    O, lse = A.attention_rows(q, K, V, 0.7)
    assert np.allclose(O, np.repeat(V, 3, axis=0), atol=1e-15)
    assert np.allclose(lse, 0.7 * (q @ K[0]), atol=1e-14)


def test_p7_equal_scores_give_mean_and_log_n():
    r = rng(7)
    N = 13
    K = r.normal(size=(N, 8))
    V = r.normal(size=(N, 8))
    O, lse = A.attention_rows(np.zeros((1, 8)), K, V, 1.0)
    assert np.allclose(O[0], V.mean(axis=0), atol=1e-14)
    assert abs(lse[0] - math.log(N)) < 1e-14
    # a constant shift of every score shifts the LSE and leaves O unchanged
    K2 = np.zeros((N, 8)); K2[:, 0] = 1.0
    q2 = np.zeros((1, 8)); q2[0, 0] = 2.5
    O2, lse2 = A.attention_rows(q2, K2, V, 1.0)
    assert np.allclose(O2[0], V.mean(axis=0), atol=1e-14)
    assert abs(lse2[0] - (2.5 + math.log(N))) < 1e-13


def test_p7_causal_row0_and_dominant_key_and_convex_hull():
    r = rng(8)
    N, d = 10, 8
    q = r.normal(size=(1, 1, N, d))
    k = r.normal(size=(1, 1, N, d))
    v = r.normal(size=(1, 1, N, d))
    O, lse = A.prefill(q, k, v, 0.4, causal=True)
    assert np.allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.4 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14
    # dominant key: scores of key 3 far above the rest
    K = r.normal(size=(N, d)) * 0.01
    K[3] = 50.0 * np.ones(d)
    Od, _ = A.attention_rows(np.ones((1, d)), K, v[0, 0], 1.0)
    assert np.allclose(Od[0], v[0, 0, 3], atol=1e-12)
    # every output row is a convex combination of V rows: with V = I it is the
    # probability row itself (non-negative, sums to 1)
    P, _ = A.attention_rows(r.normal(size=(5, d)), r.normal(size=(N, d)), np.eye(N), 0.5)
    assert (P >= 0).all() and np.allclose(P.sum(axis=1), 1.0, atol=1e-14)


def test_p7_no_visible_key_gives_zero_and_minus_inf():
    O, lse = A.attention_rows(np.ones((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert (O == 0).all() and lse[0] == -np.inf
    O, lse = A.decode_contiguous(np.ones((1, 2, 4)), np.ones((1, 1, 3, 4)), np.ones((1, 1, 3, 4)),
                                 np.array([0]), 1.0)
    assert (O == 0).all() and (lse == -np.inf).all()


# --------------------------------------------------------------------------
# P8: merging partial results of disjoint key ranges
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cuts", [[0, 40], [0, 1, 40], [0, 7, 8, 21, 40], [0, 13, 13, 40]])
def test_p8_merge_of_exact_chunks_equals_whole_row(cuts):
    r = rng(9)
    q = r.normal(size=(1, 16))
    K = r.normal(size=(40, 16)) * 2
    V = r.normal(size=(40, 16))
    O_ref, lse_ref = A.attention_rows(q, K, V, 0.3)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = A.attention_rows(q, K[a:b], V[a:b], 0.3)
        parts.append((o[0], l[0]))
    O_m, lse_m = OL.merge_partials(parts)
    assert np.allclose(O_m, O_ref[0], atol=1e-14)
    assert abs(lse_m - lse_ref[0]) < 1e-13


# --------------------------------------------------------------------------
# P9: library cross-check and brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 1)])
def test_p9_matches_torch_sdpa_math_fp64(causal, Hq, Hkv):
    torch.manual_seed(11)
    B, N, d = 2, 9, 16
    q = torch.randn(B, Hq, N, d, dtype=torch.float64)
    k = torch.randn(B, Hkv, N, d, dtype=torch.float64)
    v = torch.randn(B, Hkv, N, d, dtype=torch.float64)
    n_rep = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(n_rep, 1), v.repeat_interleave(n_rep, 1), is_causal=causal)
    O, _ = A.prefill(q, k, v, 1 / math.sqrt(d), causal=causal)
    assert np.max(np.abs(O - ref.numpy())) < 1e-12


def _brute(q, k, v, scale, causal):
    """Pure-Python loops with math.exp, straight from the definition."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = [[[[0.0] * d for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[0.0] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk) if not causal or j <= i + Nk - Nq]
                s = {j: scale * sum(float(q[b, h, i, c]) * float(k[b, g, j, c]) for c in range(d)) for j in keys}
                mx = max(s.values())
                z = sum(math.exp(s[j] - mx) for j in keys)
                for c in range(d):
                    O[b][h][i][c] = sum(math.exp(s[j] - mx) / z * float(v[b, g, j, c]) for j in keys)
                L[b][h][i] = mx + math.log(z)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("Nq,Nk,causal", [(3, 3, True), (2, 5, True), (4, 3, False)])
def test_p9_brute_force_tiny(Nq, Nk, causal):
    q, k, v = make_prefill_inputs(1, 4, 2, Nq, Nk, 3, "bf16", 12)
    O, lse = A.prefill(q, k, v, 0.6, causal)
    Ob, lseb = _brute(A._f64(q), A._f64(k), A._f64(v), 0.6, causal)
    assert np.max(np.abs(O - Ob)) < 1e-14 and np.max(np.abs(lse - lseb)) < 1e-13


def test_mask_alignment_bottom_right_vs_sdpa_top_left():
    g = golden("sdpa_top_left_pitfall.json")
    torch.manual_seed(0)
    q = torch.randn(1, 1, g["Nq"], 8, dtype=torch.float64)
    k = torch.randn(1, 1, g["Nk"], 8, dtype=torch.float64)
    v = torch.randn(1, 1, g["Nk"], 8, dtype=torch.float64)
    y = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    assert torch.allclose(y, v[:, :, :g["top_left_visible_keys"]])      # the pitfall, as printed
    O, _ = A.prefill(q, k, v, 8 ** -0.5, causal=True)
    assert A.causal_key_limit(0, g["Nq"], g["Nk"]) == g["bottom_right_visible_keys"]
    O_nc, _ = A.prefill(q, k, v, 8 ** -0.5, causal=False)
    assert np.allclose(O, O_nc, atol=1e-15) and not np.allclose(O, y.numpy())


# --------------------------------------------------------------------------
# Planted mistakes: each plausible bug in a copy of the oracle fails a pin
# --------------------------------------------------------------------------
def _mutant_rows(kind):
    def rows(q_rows, K, V, scale, key_limits=None, key_starts=None):
        q_rows, K, V = A._f64(q_rows), A._f64(K), A._f64(V)
        R, Nk = q_rows.shape[0], K.shape[0]
        S = (q_rows @ K.T) * (1.0 if kind == "no_scale" else scale)
        if key_limits is not None:
            lim = np.asarray(key_limits).reshape(R, 1)
            if kind == "mask_off_by_one":
                lim = lim - 1
            S = np.where(np.arange(Nk)[None, :] < lim, S, -np.inf)
        if key_starts is not None:
            S = np.where(np.arange(Nk)[None, :] >= np.asarray(key_starts).reshape(R, 1), S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        ell = E.sum(axis=1, keepdims=True)
        if kind == "no_normalise":
            O = E @ V
        elif kind == "transposed_v":
            O = (E / ell) @ V[::-1]
        else:
            O = (E / ell) @ V
        lse = (m + (ell if kind == "lse_no_log" else np.log(ell)))[:, 0]
        return O, lse
    return rows


@pytest.mark.parametrize("kind", ["no_scale", "mask_off_by_one", "no_normalise", "transposed_v", "lse_no_log"])
def test_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(A, "attention_rows", _mutant_rows(kind))
    checks = [test_p1_worked_example_pins_oracle_lse,
              lambda: test_p9_matches_torch_sdpa_math_fp64(True, 4, 2),
              lambda: test_p9_brute_force_tiny(2, 5, True),
              test_p7_equal_scores_give_mean_and_log_n]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"planted mistake {kind!r} passed every pin"


def test_planted_tile_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    with pytest.raises(AssertionError):
        test_p9_matches_torch_sdpa_math_fp64(False, 4, 2)
