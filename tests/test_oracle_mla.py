"""Pins of the MLA decode oracle (CPU only).

The cache-size numbers the pages print fix the latent layout; the absorption
identity fixes the latent-space decode against MLA built head by head from the
page's equations (reconstructed keys and values, decoupled position key,
scale over the combined width); closed forms and planted mistakes do the rest.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla as M
from oracle import attention as A

from conftest import GOLDEN


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_printed_cache_sizes():
    g = golden("mla_cache.json")
    d = g["demo"]
    head_dim = d["embed_dim"] // d["num_heads"]
    assert M.mla_cache_numbers(d["kv_latent_dim"], d["rope_dim"]) == d["cached_numbers"]
    assert M.mha_cache_numbers(d["num_heads"], head_dim) == d["mha_numbers"]
    v2 = g["deepseek_v2"]
    assert M.mla_cache_numbers(v2["d_c"], v2["d_r"]) == v2["mla_numbers"]
    assert M.mha_cache_numbers(v2["heads"], v2["head_dim"]) == v2["mha_numbers"]
    assert M.equivalent_gqa_groups(v2["d_c"], v2["d_r"], v2["head_dim"]) == v2["gqa_groups"]
    v3 = g["deepseek_v3"]
    mla_b = M.mla_cache_numbers(v3["d_c"], v3["d_r"], v3["layers"]) * v3["bytes_per_elem"]
    mha_b = M.mha_cache_numbers(v3["heads"], v3["head_dim"], v3["layers"]) * v3["bytes_per_elem"]
    assert mla_b == v3["mla_bytes_per_token"]
    assert round(mha_b / 2 ** 20, 1) == v3["mha_mib_per_token"]
    assert round(mha_b / mla_b) == v3["ratio"]


def _model(seed, B=2, H=4, d_head=16, d_c=24, d_r=8, S=40, lens=(17, 40)):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)
    return dict(q_c=r(B, H, d_head), q_r=r(B, H, d_r), w_uk=r(H, d_head, d_c) / math.sqrt(d_c),
                w_uv=r(H, d_head, d_c) / math.sqrt(d_c), latent=r(B, S, d_c), k_rope=r(B, S, d_r),
                lens=torch.tensor(lens, dtype=torch.int32), scale=1 / math.sqrt(d_head + d_r), d_c=d_c)


def _absorbed(m):
    q = np.concatenate([M.absorb_query(m["q_c"], m["w_uk"]), m["q_r"].numpy()], axis=2)
    kv = np.concatenate([m["latent"].numpy(), m["k_rope"].numpy()], axis=2)
    O_lat, lse = M.mla_decode_latent(q, kv, m["lens"], m["scale"], m["d_c"])
    return M.latent_to_head(O_lat, m["w_uv"]), lse


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorption_identity(seed):
    m = _model(seed)
    Oe, le = M.mla_decode_explicit(m["q_c"], m["q_r"], m["w_uk"], m["w_uv"], m["latent"], m["k_rope"], m["lens"],
                                   m["scale"])
    Oa, la = _absorbed(m)
    np.testing.assert_allclose(Oa, Oe, rtol=0, atol=1e-12)
    np.testing.assert_allclose(la, le, rtol=0, atol=1e-12)


def test_absorbed_content_scores_at_fp32_are_within_rounding():
    """The page's check in fp32: explicit and absorbed content scores differ
    by float32 rounding only (it prints 2.98e-07 for its model)."""
    m = _model(3)
    qc, wuk, c = m["q_c"].float(), m["w_uk"].float(), m["latent"].float()
    kc = torch.einsum("hec,bsc->bhse", wuk, c)
    explicit = torch.einsum("bhe,bhse->bhs", qc, kc)
    absorbed = torch.einsum("bhc,bsc->bhs", torch.einsum("bhe,hec->bhc", qc, wuk), c)
    diff = (explicit - absorbed).abs().max().item()
    assert 0 < diff < 100 * golden("mla_cache.json")["absorption_max_abs_diff_fp32"]


def test_single_cached_token_closed_form():
    m = _model(4, lens=(1, 1))
    Oe, le = M.mla_decode_explicit(m["q_c"], m["q_r"], m["w_uk"], m["w_uv"], m["latent"], m["k_rope"], m["lens"],
                                   m["scale"])
    for b in range(2):
        for h in range(4):
            c = m["latent"][b, 0].numpy()
            k = np.concatenate([m["w_uk"][h].numpy() @ c, m["k_rope"][b, 0].numpy()])
            q = np.concatenate([m["q_c"][b, h].numpy(), m["q_r"][b, h].numpy()])
            np.testing.assert_allclose(le[b, h], (q @ k) / math.sqrt(16 + 8), atol=1e-13)
            np.testing.assert_allclose(Oe[b, h], m["w_uv"][h].numpy() @ c, atol=1e-13)


def test_paged_latent_cache_equals_contiguous():
    m = _model(5)
    q = np.concatenate([M.absorb_query(m["q_c"], m["w_uk"]), m["q_r"].numpy()], axis=2)
    kv = torch.cat([m["latent"], m["k_rope"]], dim=2)           # (B, S, w)
    bs, B, S = 4, 2, 40
    nb = B * S // bs
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(6))
    pool = torch.zeros(nb, bs, kv.shape[2], dtype=torch.float64)
    table = torch.full((B, S // bs), -1, dtype=torch.int32)
    for b in range(B):
        for j in range(S // bs):
            blk = int(perm[b * (S // bs) + j])
            table[b, j] = blk
            pool[blk] = kv[b, j * bs:(j + 1) * bs]
    Oc, lc = M.mla_decode_latent(q, kv, m["lens"], m["scale"], m["d_c"])
    Op, lp = M.mla_decode_latent(q, pool, m["lens"], m["scale"], m["d_c"], table, bs)
    np.testing.assert_array_equal(Op, Oc)
    np.testing.assert_array_equal(lp, lc)


def test_planted_untransposed_absorption_is_caught(monkeypatch):
    # absorbing with W^UK instead of W^UK^T needs d_head == d_c to even run
    monkeypatch.setattr(M, "absorb_query", lambda q_c, w_uk: np.einsum("bhe,hce->bhc", A._f64(q_c), A._f64(w_uk)))
    with pytest.raises(AssertionError):
        m = _model(7, d_head=24, d_c=24)
        Oe, _ = M.mla_decode_explicit(m["q_c"], m["q_r"], m["w_uk"], m["w_uv"], m["latent"], m["k_rope"],
                                      m["lens"], m["scale"])
        Oa, _ = _absorbed(m)
        np.testing.assert_allclose(Oa, Oe, rtol=0, atol=1e-12)


def test_planted_value_without_latent_prefix_is_caught(monkeypatch):
    real = M.attention_rows
    monkeypatch.setattr(M, "attention_rows", lambda q, K, V, s, *a: real(q, K, K[:, -V.shape[1]:], s, *a))
    with pytest.raises(AssertionError):
        test_absorption_identity(0)
