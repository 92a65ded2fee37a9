"""Pins of the FP8 (E4M3) cache oracle (CPU only).

The code -> value table is checked against the E4M3 values PyTorch's
float8_e4m3fn type assigns to every byte, and against closed forms; the
quantiser against PyTorch's round-to-nearest-even cast, the midpoints
between neighbouring values (ties go to the even code), saturation and a
round trip; decode against an FP8 cache against the pinned decode over the
decoded values.  The last tests plant mistakes and show that a pin catches
each.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from flashattention_kv_cache_amd.workloads import make_decode_inputs


def torch_values(codes):
    return torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_table_matches_float8_e4m3fn_for_every_byte():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = F.decode_codes(codes), torch_values(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.isnan(ours).sum() == 2                       # 0x7F and 0xFF only


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 / 8 * 2.0 ** -6),
                                        (0x08, 2.0 ** -6), (0x30, 0.5), (0x38, 1.0), (0x40, 2.0),
                                        (0x7E, 448.0), (0xC0, -2.0), (0xFE, -448.0), (0x80, -0.0)])
def test_closed_form_codes(code, value):
    assert F.e4m3_value(code) == value
    assert F.quantize_e4m3([value], 1.0)[0] == code


@pytest.mark.parametrize("scale", [1.0, 0.015625, 0.37, 3.0])
def test_quantiser_matches_round_to_nearest_even_cast(scale):
    g = torch.Generator().manual_seed(int(scale * 1000))
    x = torch.randn(20000, generator=g) * (100 * scale)
    x = x[(x / scale).abs() < 440]
    ref = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.quantize_e4m3(x, scale), ref)


def test_ties_go_to_the_even_code():
    vals = F.decode_codes(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact in fp32
    codes = F.quantize_e4m3(mids.astype(np.float32), 1.0)
    assert (codes % 2 == 0).all()
    assert np.array_equal(codes, np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F)))
    assert np.array_equal(F.quantize_e4m3(-mids.astype(np.float32), 1.0), codes | 0x80)


def test_saturation_and_nan():
    assert list(F.quantize_e4m3([449.0, 464.0, 1e6, -500.0, -1e30], 1.0)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert F.quantize_e4m3([900.0], 2.0)[0] == 0x7E
    assert F.quantize_e4m3([float("nan")], 1.0)[0] & 0x7F == 0x7F


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for s in (1.0, 0.25, 8.0):
        assert np.array_equal(F.quantize_e4m3(F.decode_codes(codes) * s, s), codes)


def test_decode_fp8_is_decode_over_the_decoded_cache():
    di = make_decode_inputs(3, 8, 2, 16, "bf16", 21, seq_lens=[1, 9, 40], paged=True, block_size=4)
    g = torch.Generator().manual_seed(5)
    kc = (torch.randn(di.k_cache.shape, generator=g) * 30).to(torch.float8_e4m3fn).view(torch.uint8)
    vc = (torch.randn(di.v_cache.shape, generator=g) * 30).to(torch.float8_e4m3fn).view(torch.uint8)
    ks, vs = 1 / 32, 0.05
    O, lse = F.decode_fp8(di.q, kc, vc, di.seq_lens, 0.25, ks, vs, di.block_table, 4)
    Kf = kc.view(torch.float8_e4m3fn).to(torch.float64) * ks
    Vf = vc.view(torch.float8_e4m3fn).to(torch.float64) * vs
    Or, lr = oracle.decode_paged(di.q, Kf, Vf, di.block_table, di.seq_lens, 4, 0.25)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(lse, lr)


def test_append_fp8_places_quantised_rows():
    from flashattention_kv_cache_amd.workloads import make_chunked_inputs
    ci = make_chunked_inputs(2, 4, 2, 16, "bf16", 22, chunk=5, past_lens=[3, 14], block_size=4)
    kc = torch.zeros(ci.k_cache.shape, dtype=torch.uint8)
    vc = torch.zeros(ci.v_cache.shape, dtype=torch.uint8)
    k2, v2 = F.append_fp8(kc, vc, ci.block_table, ci.seq_lens, ci.k_new, ci.v_new, 4, 0.5, 0.25)
    for b in range(2):
        L = int(ci.seq_lens[b])
        for i, t in enumerate(range(L - 5, L)):
            blk, slot = int(ci.block_table[b, t // 4]), t % 4
            for g in range(2):
                assert np.array_equal(k2[blk, slot, g], F.quantize_e4m3(ci.k_new[b, g, i], 0.5))
                assert np.array_equal(v2[blk, slot, g], F.quantize_e4m3(ci.v_new[b, g, i], 0.25))


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------
def test_planted_fnuz_bias_is_caught(monkeypatch):
    table = np.array([F.e4m3_value(c) / 2 for c in range(256)])  # exponent bias 8
    monkeypatch.setattr(F, "_TABLE", table)
    with pytest.raises(AssertionError):
        test_table_matches_float8_e4m3fn_for_every_byte()


def test_planted_truncation_is_caught(monkeypatch):
    real = F.quantize_e4m3

    def truncating(x, scale):
        q = (np.asarray(F._f64(x), dtype=np.float32) / np.float32(scale)).astype(np.float64)
        vals = F._TABLE[F._POS]
        a = np.minimum(np.abs(q), F.E4M3_MAX)
        code = np.searchsorted(vals, a, side="right") - 1
        return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)

    monkeypatch.setattr(F, "quantize_e4m3", truncating)
    with pytest.raises(AssertionError):
        test_quantiser_matches_round_to_nearest_even_cast(0.37)
    monkeypatch.setattr(F, "quantize_e4m3", real)
