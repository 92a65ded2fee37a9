"""FP8 KV cache on the CPU (test infrastructure only).

The pages give one fact about it: the cache may store one byte per number in
FP8 instead of two in BF16, which halves its size and the bytes a decode step
reads ("Генерация и KV-кэш", section "Сколько весит KV-кэш": bytes per
number 2 in FP16/BF16, 1 in FP8, and the table of levers that lists an FP8
cache).  Everything else is a reading taken here, because the pages are
silent on it:

* format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN;
  there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448;
* scaling: one fp32 scale per tensor (one for K, one for V); the number a
  code stands for is decode(code) * scale;
* quantisation (the append of bf16 keys and values into an FP8 cache): the
  fp32 quotient x / scale (IEEE division) rounded to the nearest E4M3 value,
  ties to the even code, with magnitudes beyond 448 saturated to 448; a NaN
  stays NaN.

Decode against an FP8 cache is the decode of the pinned definition
(oracle.attention) applied to the decoded values.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, decode_contiguous, decode_paged

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The number an E4M3 code (0..255) stands for, from the bit layout."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# the finite non-negative codes, in increasing order of value (codes 0x00..0x7E)
_POS = np.arange(0x7F)


def decode_codes(codes) -> np.ndarray:
    """Array of E4M3 codes (uint8, any shape; torch or numpy) -> fp64 values."""
    try:
        import torch
        if isinstance(codes, torch.Tensor):
            codes = codes.detach().cpu().view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize_e4m3(x, scale: float) -> np.ndarray:
    """Codes (uint8) of x / scale: the quotient is formed in fp32, rounded to
    the nearest E4M3 value with ties to the even code, saturated at 448."""
    q = (np.asarray(_f64(x), dtype=np.float32) / np.float32(scale)).astype(np.float64)
    vals = _TABLE[_POS]                                   # 0, 2^-9, ..., 448 (increasing)
    nan = np.isnan(q)
    a = np.minimum(np.abs(np.where(nan, 0.0, q)), E4M3_MAX)
    hi = np.minimum(np.searchsorted(vals, a), len(vals) - 1)   # vals[hi-1] < a <= vals[hi]
    lo = np.maximum(hi - 1, 0)
    dl, dh = a - vals[lo], vals[hi] - a
    tie_even = np.where(lo % 2 == 0, lo, hi)
    code = np.where(dh < dl, hi, np.where(dl < dh, lo, tie_even))
    code = np.where(vals[hi] == a, hi, code)
    neg = np.signbit(q) & ~nan
    out = (code | np.where(neg, 0x80, 0)).astype(np.uint8)
    out[nan] = 0x7F
    return out


class _Decoded:
    """A cache of codes seen as the numbers they stand for, decoded on access
    (value(code) * scale), so that a multi-GiB cache is never expanded whole."""

    def __init__(self, codes, scale: float):
        self.codes = _codes(codes)
        self.scale = float(scale)
        self.shape = self.codes.shape

    def __getitem__(self, idx):
        return decode_codes(self.codes[idx]) * self.scale


def decode_fp8(q, k_codes, v_codes, seq_lens, scale: float, k_scale: float, v_scale: float,
               block_table=None, block_size: int = 0, heads=None, window: int = 0):
    """Decode against an FP8 cache: the caches hold E4M3 codes (contiguous
    (B, Hkv, S_cap, d) or a paged pool (num_blocks, block_size, Hkv, d)); their
    values are decode(code) * k_scale and decode(code) * v_scale."""
    K = _Decoded(k_codes, k_scale)
    V = _Decoded(v_codes, v_scale)
    if block_table is None:
        return decode_contiguous(q, K, V, seq_lens, scale, heads=heads, window=window)
    return decode_paged(q, K, V, block_table, seq_lens, block_size, scale, heads=heads, window=window)


def append_fp8(k_cache, v_cache, block_table, seq_lens, k_new, v_new, block_size: int,
               k_scale: float, v_scale: float):
    """The batched append into an FP8 cache: new rows (B, Hkv, n, d) are
    quantised with ``quantize_e4m3`` and written like ``paged.append_batch``
    (contiguous caches when block_table is None).  Returns the new code arrays
    (uint8 numpy)."""
    from .paged import append_batch, append_batch_contiguous
    kc = np.array(_codes(k_cache), copy=True)
    vc = np.array(_codes(v_cache), copy=True)
    kq = quantize_e4m3(k_new, k_scale)
    vq = quantize_e4m3(v_new, v_scale)
    if block_table is None:
        return append_batch_contiguous(kc, vc, seq_lens, kq, vq)
    return append_batch(kc, vc, block_table, seq_lens, kq, vq, block_size)


def _codes(t):
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().cpu().view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.uint8)
