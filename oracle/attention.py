"""Plain fp64 definition of exact softmax attention (test infrastructure only).

What is computed, and where the pages say so:

* Scores and softmax: softmax(Q K^T / sqrt(d_k)) V, unchanged by GQA
  ("Module 09: Efficient Attention", section "The Math: Sharing Keys and
  Values"; "Генерация и KV-кэш", section "KV-кэш для одной головы на NumPy",
  where the scores are divided by sqrt(d) and the row maximum is subtracted
  before exponentiating).  The scale is a parameter; the workloads pass
  1/sqrt(d).
* GQA head mapping: query head h reads key/value head floor(h / n_rep) with
  n_rep = H_q / H_kv, i.e. repeat_interleave, not repeat/tile ("Module 09",
  "The Math: Sharing Keys and Values" and "Common Pitfalls" items 2-3).
* Causal mask: a lower-triangular mask when N_q = N_k ("Генерация и KV-кэш",
  NumPy listing ``full_causal``); when queries extend a non-empty cache the mask
  is aligned to the bottom-right corner ("Генерация и KV-кэш", "Три ловушки"
  item 2).  Reading taken: key j is visible to query i iff
  j <= i + (N_k - N_q).
* Decode: one new query against every cached key, itself included, with no
  mask ("Генерация и KV-кэш", NumPy decode step).  The cache already holds the
  new token; ``seq_lens`` counts it.
* Sliding window: with a window of W keys, a (causal) query sees only the W
  most recent keys, itself included ("Module 09: Efficient Attention",
  section "Attention Mask Gallery": the printed window-3 mask over six
  positions, where row i attends keys i-2 .. i).  Aligned like the causal
  mask: query i sees keys j with i + (N_k - N_q) - W < j <= i + (N_k - N_q).
  W = 0 means no window.
* Paged read: token t of a sequence lives at
  pool[block_table[t // block_size], t % block_size] ("Module 09", "Code: A
  Paged KV Cache from Scratch").
* LSE (not on the pages; reading taken): natural log of the sum of exp of the
  scaled, unmasked scores, = row max + ln(row sum).

Materialisation: the scores of one (b, h) are formed a block of whole rows at
a time, and each row gets an ordinary two-pass softmax (max, then exp / sum).
There is no streaming over keys here.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor or array (fp32/bf16) to fp64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head h: floor(h / (Hq / Hkv))."""
    if Hq % Hkv:
        raise ValueError("num_kv_heads must divide num_heads")
    return h // (Hq // Hkv)


def causal_key_limit(i: int, Nq: int, Nk: int) -> int:
    """Number of keys visible to query row i under the bottom-right causal mask."""
    return min(Nk, max(0, i + (Nk - Nq) + 1))


def window_key_start(i: int, Nq: int, Nk: int, window: int) -> int:
    """First key visible to query row i under a sliding window of ``window``
    keys aligned to the bottom-right corner (0 when window == 0)."""
    if window <= 0:
        return 0
    return max(0, i + (Nk - Nq) - window + 1)


def attention_rows(q_rows, K, V, scale: float, key_limits=None, key_starts=None):
    """Attention of R query rows against one head's keys.

    q_rows (R, d), K and V (Nk, d); keys ``key_starts[r] <= j < key_limits[r]``
    are visible to row r (a prefix when key_starts is None, all keys when both
    are None).  Returns O (R, d) and LSE (R,) in fp64.  A row with no visible
    key gets O = 0 and LSE = -inf.
    """
    q_rows, K, V = _f64(q_rows), _f64(K), _f64(V)
    R, Nk = q_rows.shape[0], K.shape[0]
    S = scale * (q_rows @ K.T)                          # (R, Nk) scores
    if key_limits is not None:
        lim = np.asarray(key_limits, dtype=np.int64).reshape(R, 1)
        S = np.where(np.arange(Nk)[None, :] < lim, S, -np.inf)
    if key_starts is not None:
        lo = np.asarray(key_starts, dtype=np.int64).reshape(R, 1)
        S = np.where(np.arange(Nk)[None, :] >= lo, S, -np.inf)
    O = np.zeros((R, V.shape[1]))
    lse = np.full(R, -np.inf)
    live = np.isfinite(S).any(axis=1)
    if live.any():
        Sl = S[live]
        m = Sl.max(axis=1, keepdims=True)                # pass 1: row max
        E = np.exp(Sl - m)                               # pass 2: exponentials
        ell = E.sum(axis=1, keepdims=True)
        O[live] = (E / ell) @ V
        lse[live] = (m + np.log(ell))[:, 0]
    return O, lse


def prefill(q, k, v, scale: float, causal: bool, row_block: int = 1024, window: int = 0):
    """Full prefill: q (B, Hq, Nq, d), k and v (B, Hkv, Nk, d); ``window`` > 0
    adds the sliding-window lower bound to the causal mask.

    Returns O (B, Hq, Nq, d) and LSE (B, Hq, Nq), fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Nq, v.shape[3]))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for r0 in range(0, Nq, row_block):
                rows = range(r0, min(Nq, r0 + row_block))
                lim = [causal_key_limit(i, Nq, Nk) for i in rows] if causal else None
                st = [window_key_start(i, Nq, Nk, window) for i in rows] if window else None
                o, l = attention_rows(q[b, h, r0:r0 + len(rows)], k[b, g], v[b, g], scale, lim, st)
                O[b, h, r0:r0 + len(rows)] = o
                lse[b, h, r0:r0 + len(rows)] = l
    return O, lse


def prefill_rows(q, k, v, scale: float, causal: bool, rows, window: int = 0):
    """Selected output rows of a prefill, one by one: ``rows`` is a list of
    (b, h, i).  Returns O (R, d) and LSE (R,).  Used to check full-size runs
    whose whole output the oracle cannot afford."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((len(rows), v.shape[3]))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        g = kv_head_of(h, Hq, Hkv)
        lim = causal_key_limit(i, Nq, Nk) if causal else Nk
        st = window_key_start(i, Nq, Nk, window)
        o, l = attention_rows(_f64(q[b, h, i:i + 1]), _f64(k[b, g, st:lim]), _f64(v[b, g, st:lim]), scale)
        O[r], lse[r] = o[0], l[0]
    return O, lse


def paged_gather(pool, table_row, L: int, g: int, block_size: int):
    """Rows 0..L-1 of KV head g of one sequence, read through its block table:
    token t comes from pool[table_row[t // block_size], t % block_size, g]
    (one indexed read of all L tokens, written as that formula)."""
    if L == 0:
        return np.zeros((0, pool.shape[-1]))
    t = np.arange(L)
    blk = _i64(table_row)[t // block_size]
    return _f64(pool[blk, t % block_size, g])


def decode_contiguous(q, k_cache, v_cache, seq_lens, scale: float, heads=None, window: int = 0):
    """One new query per (b, h) against the first L_b cached keys (the last
    ``window`` of them when window > 0).

    q (B, Hq, d); caches (B, Hkv, S_cap, d).  ``heads`` optionally restricts
    the work to a list of (b, h).  Returns O (B, Hq, d) and LSE (B, Hq) (rows
    not computed are left NaN)."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    lens = _i64(seq_lens)
    O = np.full((B, Hq, v_cache.shape[-1]), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        g = kv_head_of(h, Hq, Hkv)
        L = int(lens[b])
        st = window_key_start(0, 1, L, window)
        o, l = attention_rows(_f64(q[b, h:h + 1]), _f64(k_cache[b, g, st:L]), _f64(v_cache[b, g, st:L]), scale)
        O[b, h], lse[b, h] = o[0], l[0]
    return O, lse


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, block_size: int, scale: float, heads=None,
                 window: int = 0):
    """Decode against a paged cache: pools (num_blocks, block_size, Hkv, d),
    block_table (B, max_blocks).  Same outputs as ``decode_contiguous``."""
    B, Hq, d = q.shape
    Hkv = k_pool.shape[2]
    lens = _i64(seq_lens)
    table = _i64(block_table)
    O = np.full((B, Hq, v_pool.shape[-1]), np.nan)
    lse = np.full((B, Hq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    cache = {}
    for b, h in todo:
        g = kv_head_of(h, Hq, Hkv)
        L = int(lens[b])
        if (b, g) not in cache:
            cache[(b, g)] = (paged_gather(k_pool, table[b], L, g, block_size),
                             paged_gather(v_pool, table[b], L, g, block_size))
        K, V = cache[(b, g)]
        st = window_key_start(0, 1, L, window)
        o, l = attention_rows(_f64(q[b, h:h + 1]), K, V, scale, None, [st])
        O[b, h], lse[b, h] = o[0], l[0]
    return O, lse
