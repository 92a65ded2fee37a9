"""The pages' streaming (online) softmax, in fp64 — test infrastructure only.

This is not how the oracle produces expected values (``attention`` does that
with a materialised two-pass softmax).  It exists to pin that definition: the
two must agree to fp64 rounding, which the lecture notes give as about 1e-15
("Li Hongyi, Machine Learning 2026: FlashAttention, KV cache and positional
embeddings", section "Что сделать руками", exercise 1).

Notation follows the same notes, lecture "Ускоряем генерацию, часть 1:
FlashAttention", passage "Трюк: сначала ошибёмся, потом поправим": scores a_i
arrive in blocks; after block k the running maximum is d_k, the running sum of
exponentials is s_k, and the running (already normalised) output is O_k:

    d_k = max(d_{k-1}, max_{i in block k} a_i)
    s_k = s_{k-1} e^{d_{k-1} - d_k} + sum_{i in block k} e^{a_i - d_k}
    O_k = O_{k-1} (s_{k-1} / s_k) e^{d_{k-1} - d_k} + sum_{i in block k} (e^{a_i - d_k} / s_k) v_i

with d_0 = -inf, s_0 = 0, O_0 = 0 (the first block's correction factor is 0,
as in the tiled listing of "KV Cache, Flash Attention and Inference
Optimization", step 2 "tiled softmax", which sets the old-exponential factor to
0 while the running max is -inf).
"""
from __future__ import annotations

import math

import numpy as np


def online_softmax_stats(a, block: int):
    """Run the (d_k, s_k) recurrence over scores ``a`` in blocks of ``block``.

    Returns the list of (d_k, s_k) after each block; the last pair gives
    max_i a_i and sum_i e^{a_i - max}."""
    a = [float(x) for x in a]
    d_prev, s_prev = -math.inf, 0.0
    out = []
    for start in range(0, len(a), block):
        blk = a[start:start + block]
        d_k = max(d_prev, max(blk))
        corr = math.exp(d_prev - d_k) if d_prev != -math.inf else 0.0
        s_k = s_prev * corr + sum(math.exp(x - d_k) for x in blk)
        out.append((d_k, s_k))
        d_prev, s_prev = d_k, s_k
    return out


def online_attention_row(q, K, V, scale: float, block: int):
    """One query row streamed over its keys in blocks, with the normalised
    output recurrence O_k above.  Returns (O, lse) with lse = d_K + ln s_K."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d_prev, s_prev = -math.inf, 0.0
    O = np.zeros(V.shape[1])
    for start in range(0, K.shape[0], block):
        a = scale * (K[start:start + block] @ q)          # this block's scores
        d_k = max(d_prev, float(a.max()))
        corr = math.exp(d_prev - d_k) if d_prev != -math.inf else 0.0
        e = np.exp(a - d_k)
        s_k = s_prev * corr + float(e.sum())
        O = O * (s_prev / s_k) * corr + (e / s_k) @ V[start:start + block]
        d_prev, s_prev = d_k, s_k
    if s_prev == 0.0:
        return O, -math.inf
    return O, d_prev + math.log(s_prev)


def merge_partials(parts):
    """Merge partial results of disjoint key ranges of one query row.

    Each part is (O_s, lse_s): the exact normalised output over its keys and
    the log of its sum of exponentials.  Writing lse_s = d_s + ln s_s, folding
    part after part is the O_k recurrence above with a whole part standing in
    for one block (this merge is not on the pages; it is that recurrence
    applied to two finished states):

        M   = max_s lse_s
        w_s = e^{lse_s - M}
        O   = sum_s w_s O_s / sum_s w_s,     lse = M + ln sum_s w_s

    Parts with lse_s = -inf (no keys) carry no weight.  Returns (O, lse)."""
    lses = np.array([float(l) for _, l in parts])
    if len(parts) == 0 or not np.isfinite(lses).any():
        dim = len(parts[0][0]) if parts else 0
        return np.zeros(dim), -math.inf
    M = lses.max()
    w = np.exp(lses - M)
    O = sum(wi * np.asarray(o, dtype=np.float64) for wi, (o, _) in zip(w, parts) if wi > 0)
    return O / w.sum(), M + math.log(w.sum())
