"""Paged KV cache on the CPU: block allocation, token append, and chunked
prefill against a cache (test infrastructure only).

What is computed, and where the pages say so:

* Pool and table: K and V live in a pool of fixed-size blocks of shape
  (num_blocks, block_size, H_kv, d); each sequence owns a list of physical
  block ids, its block table.  A free list hands blocks out and takes them
  back, so free + used is constant ("Module 09: Efficient Attention", section
  "Code: A Paged KV Cache from Scratch").  Reading taken: the free list starts
  as 0 .. num_blocks-1 and ``allocate`` takes from its end, which is what gives
  the table [7, 6] that the page prints for its 8-block pool.
* Append: token t of a sequence is written to slot
  (block_table[t // block_size], t % block_size); a new block is claimed when
  t % block_size == 0 (same section).
* Prefix sharing: two sequences may list the same physical block; a shared
  block is read by both (section "Sharing Blocks: Copy-on-Write").
* Chunked prefill: the Nq newest tokens of a sequence whose cache holds L
  tokens (the new ones included) attend to the whole sequence under the
  causal mask aligned to the bottom-right corner, i.e. query i sees keys
  j <= i + (L - Nq) ("Генерация и KV-кэш", section "Три ловушки", item 2).
  Nq = 1 is the decode step.

Values are copied, never converted, by the append: the pool keeps its dtype
and the copy is bit-exact.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _i64, attention_rows, kv_head_of, paged_gather, window_key_start


class BlockAllocator:
    """Free list over the physical blocks of one pool."""

    def __init__(self, num_blocks: int):
        self.num_blocks = int(num_blocks)
        self.free = list(range(self.num_blocks))

    def allocate(self) -> int:
        if not self.free:
            raise MemoryError("paged pool exhausted")
        return self.free.pop()

    def release(self, blk: int) -> None:
        if not 0 <= blk < self.num_blocks or blk in self.free:
            raise ValueError(f"block {blk} is not in use")
        self.free.append(blk)

    @property
    def num_free(self) -> int:
        return len(self.free)

    @property
    def num_used(self) -> int:
        return self.num_blocks - len(self.free)


class PagedSequence:
    """One sequence in a paged pool: its block table and its length."""

    def __init__(self):
        self.table: list[int] = []
        self.length = 0


def slot_of(table_row, t: int, block_size: int):
    """(physical block, slot) of token t: (table_row[t // block_size], t % block_size)."""
    return int(table_row[t // block_size]), t % block_size


def append_token(pool_k, pool_v, alloc: BlockAllocator, seq: PagedSequence, k_tok, v_tok) -> None:
    """Append one token's K and V, each (H_kv, d), to ``seq``: claim a block
    when the slot index wraps to 0, then write slot (table[t // bs], t % bs)."""
    bs = pool_k.shape[1]
    t = seq.length
    if t % bs == 0:
        seq.table.append(alloc.allocate())
    blk, slot = slot_of(seq.table, t, bs)
    pool_k[blk, slot] = k_tok
    pool_v[blk, slot] = v_tok
    seq.length = t + 1


def share_prefix(src: PagedSequence, num_blocks: int) -> PagedSequence:
    """A new sequence whose first ``num_blocks`` logical blocks are the same
    physical blocks as those of ``src`` (no block is claimed)."""
    if num_blocks < 0 or num_blocks > len(src.table):
        raise ValueError("prefix longer than the source sequence")
    s = PagedSequence()
    s.table = list(src.table[:num_blocks])
    return s


def append_batch(k_pool, v_pool, block_table, seq_lens, k_new, v_new, block_size: int):
    """The batched append: ``k_new``/``v_new`` (B, H_kv, n, d) hold n new tokens
    per sequence; ``seq_lens`` (B) are the lengths AFTER the append, so token i
    of sequence b lands at position t = L_b - n + i, i.e. in slot
    (block_table[b, t // block_size], t % block_size).  Works on copies: returns
    the new (k_pool, v_pool), same dtype and layout (torch tensors or arrays)."""
    k_out = k_pool.clone() if hasattr(k_pool, "clone") else np.array(k_pool, copy=True)
    v_out = v_pool.clone() if hasattr(v_pool, "clone") else np.array(v_pool, copy=True)
    table = _i64(block_table)
    lens = _i64(seq_lens)
    B, Hkv, n = k_new.shape[0], k_new.shape[1], k_new.shape[2]
    for b in range(B):
        start = int(lens[b]) - n
        for i in range(n):
            blk, slot = slot_of(table[b], start + i, block_size)
            for g in range(Hkv):
                k_out[blk, slot, g] = k_new[b, g, i]
                v_out[blk, slot, g] = v_new[b, g, i]
    return k_out, v_out


def append_batch_contiguous(k_cache, v_cache, seq_lens, k_new, v_new):
    """Contiguous-cache version of ``append_batch``: caches (B, H_kv, S_cap, d),
    token i of sequence b goes to row L_b - n + i."""
    k_out = k_cache.clone() if hasattr(k_cache, "clone") else np.array(k_cache, copy=True)
    v_out = v_cache.clone() if hasattr(v_cache, "clone") else np.array(v_cache, copy=True)
    lens = _i64(seq_lens)
    B, n = k_new.shape[0], k_new.shape[2]
    for b in range(B):
        start = int(lens[b]) - n
        k_out[b, :, start:start + n] = k_new[b]
        v_out[b, :, start:start + n] = v_new[b]
    return k_out, v_out


def chunked_prefill(q, k_cache, v_cache, seq_lens, scale: float, causal: bool = True,
                    block_table=None, block_size: int = 0, rows=None, window: int = 0):
    """Attention of the Nq newest tokens of each sequence against its whole
    cache.

    q (B, Hq, Nq, d); caches contiguous (B, H_kv, S_cap, d) when
    ``block_table`` is None, else paged pools (num_blocks, block_size, H_kv, d)
    with block_table (B, max_blocks).  ``seq_lens`` (B) count the cached tokens,
    the Nq new ones included (L_b >= Nq when causal).  Query i of sequence b
    sees keys j < L_b - Nq + i + 1 when causal, all L_b keys otherwise; with
    ``window`` W > 0 only keys j > L_b - Nq + i - W besides.

    Returns O (B, Hq, Nq, d) and LSE (B, Hq, Nq) in fp64; with ``rows`` (a list
    of (b, h, i)) only those rows, as O (R, d) and LSE (R,).
    """
    B, Hq, Nq, d = q.shape
    Hkv = k_cache.shape[2] if block_table is not None else k_cache.shape[1]
    lens = _i64(seq_lens)
    table = _i64(block_table) if block_table is not None else None
    kv = {}

    def keys(b, g):
        if (b, g) not in kv:
            L = int(lens[b])
            if table is None:
                kv[(b, g)] = (_f64(k_cache[b, g, :L]), _f64(v_cache[b, g, :L]))
            else:
                kv[(b, g)] = (paged_gather(k_cache, table[b], L, g, block_size),
                              paged_gather(v_cache, table[b], L, g, block_size))
        return kv[(b, g)]

    def limit(b, i):
        L = int(lens[b])
        return min(L, max(0, L - Nq + i + 1)) if causal else L

    def start(b, i):
        return window_key_start(i, Nq, int(lens[b]), window)

    if rows is not None:
        O = np.zeros((len(rows), d))
        lse = np.zeros(len(rows))
        for r, (b, h, i) in enumerate(rows):
            K, V = keys(b, kv_head_of(h, Hq, Hkv))
            o, l = attention_rows(_f64(q[b, h, i:i + 1]), K, V, scale, [limit(b, i)], [start(b, i)])
            O[r], lse[r] = o[0], l[0]
        return O, lse

    O = np.zeros((B, Hq, Nq, d))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        lim = [limit(b, i) for i in range(Nq)]
        st = [start(b, i) for i in range(Nq)]
        for h in range(Hq):
            K, V = keys(b, kv_head_of(h, Hq, Hkv))
            o, l = attention_rows(_f64(q[b, h]), K, V, scale, lim, st)
            O[b, h], lse[b, h] = o, l
    return O, lse
