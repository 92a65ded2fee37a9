"""Seeded synthetic inputs for exact-attention prefill and KV-cache decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path and the CPU oracle are fed from here,
so they always see identical bits.

Recipe (the same for every workload):
  * one ``torch.Generator`` on the CPU seeded with ``seed``;
  * Q/K/V and cache entries are i.i.d. N(0, 1) drawn in fp32, then rounded to
    bf16 with round-to-nearest-even when the workload is bf16;
  * cached lengths are integers drawn uniformly from [lo, hi], both ends
    inclusive;
  * a paged pool holds exactly sum_b ceil(L_b / block_size) blocks; physical
    block ids are a seeded random permutation of the pool, handed out in
    (sequence, logical block) order; unused block-table entries are -1;
  * cache slots that no sequence owns (the tail of a contiguous row, the
    unused slots of a sequence's last block) hold NaN, so a kernel that reads
    them poisons its output.

Layouts follow the pages' axis order: q/k/v ``(B, H, N, d)``; contiguous cache
``(B, H_kv, S_cap, d)``; paged pool ``(num_blocks, block_size, H_kv, d)``
("Module 09: Efficient Attention", section "Code: A Paged KV Cache from Scratch").
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}

# FP8 caches hold the E4M3 codes of N(0, 1) draws times FP8_SIGMA (magnitudes up
# to ~5 sigma = 320 stay below E4M3's 448); FP8_SCALE = 1 / FP8_SIGMA is the
# per-tensor scale that maps the codes back to unit variance.
FP8_SIGMA = 64.0
FP8_SCALE = 1.0 / FP8_SIGMA
FP8_NAN = 0x7F           # an E4M3 NaN code: the poison of unowned FP8 slots


_CHUNK = 1 << 24  # elements per independently seeded chunk


def _normal(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to ``dtype`` ("fp8": E4M3 codes, as uint8, of
    the draws times FP8_SIGMA, rounded to nearest even by PyTorch's cast).

    One 62-bit base seed is drawn from ``gen``; element chunk c (of a fixed
    2^24 elements) is drawn from a fresh generator seeded base + c.  The values
    therefore depend only on (gen's state, shape), not on how many threads fill
    the chunks, and multi-GiB pools are generated in parallel without an fp32
    copy of the whole tensor."""
    n = math.prod(shape)
    base = int(torch.randint(0, 2 ** 62, (1,), generator=gen, dtype=torch.int64))
    out = torch.empty(n, dtype=_DTYPES[dtype])

    def fill(c: int):
        s, e = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = torch.Generator().manual_seed(base + c)
        x = torch.randn(e - s, generator=g, dtype=torch.float32)
        if dtype == "fp8":
            out[s:e] = (x * FP8_SIGMA).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            out[s:e] = x.to(out.dtype)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        workers = min(nchunks, max(1, min(16, os.cpu_count() or 1)))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.view(*shape)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str
    seed: int
    window: int = 0     # > 0: causal sliding window of that many keys

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def unmasked_pairs(self) -> int:
        """Number of (query, key) pairs that enter the softmax, per (b, h)."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        W = self.window if self.window > 0 else self.Nk + 1
        return sum(min(self.Nk, i + off + 1) - max(0, i + off + 1 - W) for i in range(self.Nq))

    def flops(self) -> int:
        """2 flop per multiply-add, 2*d MACs per pair (QK^T and PV)."""
        return 4 * self.d * self.B * self.Hq * self.unmasked_pairs()

    def algorithmic_bytes(self) -> int:
        """Each input read once, each output written once (O plus fp32 LSE)."""
        es = 4 if self.dtype == "f32" else 2
        q = self.B * self.Hq * self.Nq * self.d * es
        kv = 2 * self.B * self.Hkv * self.Nk * self.d * es
        return q + kv + q + self.B * self.Hq * self.Nq * 4


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int
    paged: bool
    dtype: str
    seed: int
    block_size: int = 16
    window: int = 0     # > 0: only the last `window` cached keys are attended

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def kv_bytes_per_token(self) -> int:
        """Cache bytes one cached token occupies in one layer (its key and value
        for every KV head): the bytes a decode step reads per cached token."""
        return 2 * self.Hkv * self.d * (1 if self.dtype == "fp8" else _DTYPES[self.dtype].itemsize)


def prefill_inputs(w: PrefillWorkload):
    """(q, k, v) on the CPU for a prefill workload."""
    return make_prefill_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.dtype, w.seed)


def make_prefill_inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (B, Hq, Nq, d), dtype)
    k = _normal(g, (B, Hkv, Nk, d), dtype)
    v = _normal(g, (B, Hkv, Nk, d), dtype)
    return q, k, v


@dataclass
class DecodeInputs:
    q: torch.Tensor                 # (B, Hq, d)
    k_cache: torch.Tensor           # contiguous (B, Hkv, S_cap, d) or pool (nb, bs, Hkv, d)
    v_cache: torch.Tensor
    seq_lens: torch.Tensor          # (B,) int32
    block_table: Optional[torch.Tensor]  # (B, max_blocks) int32 or None
    block_size: int
    kv_capacity: int                # S_cap, or number of pool blocks
    max_seq_len: int                # host-side upper bound on seq_lens
    meta: dict = field(default_factory=dict)

    @property
    def paged(self) -> bool:
        return self.block_table is not None

    def kv_bytes(self, window: int = 0) -> int:
        """Bytes of K and V that a decode step must read: 2*Hkv*d*elem per
        attended token (the last `window` of each sequence when window > 0)."""
        es = self.k_cache.element_size()   # 1 for an FP8 cache
        Hkv, d = self.k_cache.shape[2 if self.paged else 1], self.q.shape[-1]
        lens = self.seq_lens.to(torch.int64)
        if window > 0:
            lens = lens.clamp(max=window)
        return int(lens.sum()) * 2 * Hkv * d * es


def decode_inputs(w: DecodeWorkload) -> DecodeInputs:
    return make_decode_inputs(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.seed,
                              len_range=(w.len_lo, w.len_hi), paged=w.paged,
                              block_size=w.block_size)


def make_decode_inputs(B, Hq, Hkv, d, dtype, seed, len_range=None, seq_lens=None,
                       paged=False, block_size=16, s_cap: Optional[int] = None,
                       max_blocks: Optional[int] = None, spare_blocks: int = 0) -> DecodeInputs:
    """Give either ``len_range=(lo, hi)`` (lengths drawn uniformly, inclusive)
    or ``seq_lens`` (B explicit lengths).  ``spare_blocks`` adds pool blocks
    that no sequence owns (all NaN).  dtype "fp8": bf16 queries, E4M3 caches
    (codes as uint8, scale FP8_SCALE)."""
    g = torch.Generator().manual_seed(seed)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
        max_seq_len = hi
    else:
        seq_lens = torch.tensor(list(seq_lens), dtype=torch.int64)
        assert seq_lens.numel() == B
        max_seq_len = int(seq_lens.max()) if B > 0 else 0
    q = _normal(g, (B, Hq, d), "bf16" if dtype == "fp8" else dtype)
    poison = FP8_NAN if dtype == "fp8" else float("nan")
    if not paged:
        cap = s_cap if s_cap is not None else max_seq_len
        k = _normal(g, (B, Hkv, cap, d), dtype)
        v = _normal(g, (B, Hkv, cap, d), dtype)
        for b in range(B):
            L = int(seq_lens[b])
            k[b, :, L:, :] = poison
            v[b, :, L:, :] = poison
        return DecodeInputs(q, k, v, seq_lens.to(torch.int32), None, 0, cap, max_seq_len)
    bs = block_size
    nblk = [(int(L) + bs - 1) // bs for L in seq_lens]
    total = sum(nblk) + spare_blocks
    perm = torch.randperm(total, generator=g)
    mb = max_blocks if max_blocks is not None else max(1, (max_seq_len + bs - 1) // bs)
    table = torch.full((B, mb), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]].to(torch.int32)
        off += nblk[b]
    k = _normal(g, (total, bs, Hkv, d), dtype)
    v = _normal(g, (total, bs, Hkv, d), dtype)
    for b in range(B):
        L = int(seq_lens[b])
        if L % bs:
            last = int(table[b, nblk[b] - 1])
            k[last, L % bs:] = poison
            v[last, L % bs:] = poison
    for p in perm[sum(nblk):].tolist():      # spare blocks nobody owns
        k[p] = poison
        v[p] = poison
    return DecodeInputs(q, k, v, seq_lens.to(torch.int32), table, bs, total, max_seq_len)


@dataclass
class ChunkedInputs:
    """A chunk of n new tokens per sequence, to be appended to a KV cache that
    already holds each sequence's past, then attended causally against the
    whole sequence."""
    q: torch.Tensor                 # (B, Hq, n, d)
    k_new: torch.Tensor             # (B, Hkv, n, d)
    v_new: torch.Tensor
    k_cache: torch.Tensor           # contiguous (B, Hkv, S_cap, d) or pool (nb, bs, Hkv, d); past only
    v_cache: torch.Tensor
    seq_lens: torch.Tensor          # (B,) int32: past + n, the lengths after the append
    block_table: Optional[torch.Tensor]
    block_size: int
    kv_capacity: int
    max_seq_len: int

    @property
    def paged(self) -> bool:
        return self.block_table is not None


def make_chunked_inputs(B, Hq, Hkv, d, dtype, seed, chunk, past_range=None, past_lens=None,
                        paged=True, block_size=16, s_cap: Optional[int] = None,
                        max_blocks: Optional[int] = None, spare_blocks: int = 0,
                        shared_prefix_blocks: int = 0) -> ChunkedInputs:
    """Give ``past_range=(lo, hi)`` (past lengths drawn uniformly, inclusive) or
    ``past_lens``.  The cache holds the past tokens; the slots the chunk will
    occupy, like every other slot no sequence owns, hold NaN until the append.
    ``shared_prefix_blocks`` makes sequences 1.. list the first blocks of
    sequence 0 as their own first blocks (a shared prompt)."""
    g = torch.Generator().manual_seed(seed)
    if past_lens is None:
        lo, hi = past_range
        past = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
        max_seq_len = hi + chunk
    else:
        past = torch.tensor(list(past_lens), dtype=torch.int64)
        max_seq_len = (int(past.max()) if B > 0 else 0) + chunk
    lens = past + chunk
    q = _normal(g, (B, Hq, chunk, d), dtype)
    k_new = _normal(g, (B, Hkv, chunk, d), dtype)
    v_new = _normal(g, (B, Hkv, chunk, d), dtype)
    if not paged:
        cap = s_cap if s_cap is not None else max_seq_len
        k = _normal(g, (B, Hkv, cap, d), dtype)
        v = _normal(g, (B, Hkv, cap, d), dtype)
        for b in range(B):
            k[b, :, int(past[b]):] = float("nan")
            v[b, :, int(past[b]):] = float("nan")
        return ChunkedInputs(q, k_new, v_new, k, v, lens.to(torch.int32), None, 0, cap, max_seq_len)
    bs = block_size
    sp = shared_prefix_blocks
    if sp and any(int(p) < sp * bs for p in past):
        raise ValueError("every past must cover the shared prefix blocks")
    nblk = [(int(L) + bs - 1) // bs for L in lens]
    owned = [n - (sp if b > 0 else 0) for b, n in enumerate(nblk)]
    total = sum(owned) + spare_blocks
    perm = torch.randperm(total, generator=g)
    mb = max_blocks if max_blocks is not None else max(1, (max_seq_len + bs - 1) // bs)
    table = torch.full((B, mb), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        own = perm[off:off + owned[b]].to(torch.int32)
        off += owned[b]
        if b > 0 and sp:
            table[b, :sp] = table[0, :sp]
            table[b, sp:nblk[b]] = own
        else:
            table[b, :nblk[b]] = own
    k = _normal(g, (total, bs, Hkv, d), dtype)
    v = _normal(g, (total, bs, Hkv, d), dtype)
    for b in range(B):                       # chunk slots and the unused tail: NaN
        P = int(past[b])
        for j in range(P // bs, nblk[b]):
            blk = int(table[b, j])
            s0 = P % bs if j == P // bs else 0
            k[blk, s0:] = float("nan")
            v[blk, s0:] = float("nan")
    for p in perm[sum(owned):].tolist():
        k[p] = float("nan")
        v[p] = float("nan")
    return ChunkedInputs(q, k_new, v_new, k, v, lens.to(torch.int32), table, bs, total, max_seq_len)


# The five workloads: seeds are 1000 + index.  Head layouts follow the pages'
# examples: 32 query / 8 KV heads of width 128 (Llama 3 8B style) and 64 / 8
# (Llama 3 70B style); paged blocks of 16 tokens.
C1 = PrefillWorkload("single-head non-causal fp32, N=256, d=64", 1, 1, 1, 256, 256, 64, False, "f32", 1000)
C2 = PrefillWorkload("causal GQA prefill bf16, Hq=32 Hkv=8 N=4096 d=128", 1, 32, 8, 4096, 4096, 128, True, "bf16", 1001)
C3 = DecodeWorkload("contiguous decode bf16, B=64 Hq=32 Hkv=8 d=128 L~U[1024,8192]", 64, 32, 8, 128, 1024, 8192, False, "bf16", 1002)
C4 = PrefillWorkload("long-context causal GQA prefill bf16, Hq=64 Hkv=8 N=32768 d=128", 1, 64, 8, 32768, 32768, 128, True, "bf16", 1003)
C5 = DecodeWorkload("paged decode bf16, B=128 Hq=32 Hkv=8 d=128 bs=16 L~U[512,32768]", 128, 32, 8, 128, 512, 32768, True, "bf16", 1004)
WORKLOADS = (C1, C2, C3, C4, C5)


@dataclass(frozen=True)
class ChunkedWorkload:
    """n_new-token chunks appended to paged caches, then attended causally
    against each whole sequence."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    chunk: int
    past_lo: int
    past_hi: int
    block_size: int
    dtype: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, seq_lens) -> int:
        """2 flop per multiply-add over the unmasked (query, key) pairs of every
        sequence: query i of a sequence of L keys sees L - chunk + i + 1 keys."""
        n = self.chunk
        pairs = sum(n * (int(L) - n) + n * (n + 1) // 2 for L in seq_lens)
        return 4 * self.d * self.Hq * pairs

    def append_bytes(self) -> int:
        """The append reads and writes every new K and V element once."""
        es = 4 if self.dtype == "f32" else 2
        return 2 * 2 * self.B * self.Hkv * self.chunk * self.d * es


def chunked_inputs(w: ChunkedWorkload) -> ChunkedInputs:
    return make_chunked_inputs(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.seed, chunk=w.chunk,
                               past_range=(w.past_lo, w.past_hi), paged=True, block_size=w.block_size)


# A prompt chunk of 1024 tokens per sequence against paged caches that already
# hold 1024..7168 tokens (the prefill half of a chunked-prefill serving step).
CHUNKED = ChunkedWorkload("chunked prefill bf16 vs paged cache, B=4 Hq=32 Hkv=8 d=128 chunk=1024 "
                          "past~U[1024,7168] bs=16", 4, 32, 8, 128, 1024, 1024, 7168, 16, "bf16", 1005)


# Sliding-window attention (a window of 4096 keys, Mistral-style): a long causal
# GQA prefill, and the paged decode batch above (same seed, so the same cache)
# with the window applied.
WINDOW_PREFILL = PrefillWorkload("sliding-window causal GQA prefill bf16, Hq=32 Hkv=8 N=32768 d=128 W=4096",
                                 1, 32, 8, 32768, 32768, 128, True, "bf16", 1006, window=4096)
WINDOW_DECODE = DecodeWorkload("sliding-window paged decode bf16, B=128 Hq=32 Hkv=8 d=128 bs=16 "
                               "L~U[512,32768] W=4096", 128, 32, 8, 128, 512, 32768, True, "bf16", 1004,
                               window=4096)

# The paged decode batch above with an FP8 (E4M3) cache: same lengths and block
# table (same seed), one byte per cached number.
FP8_DECODE = DecodeWorkload("paged decode, bf16 queries, FP8 E4M3 cache, B=128 Hq=32 Hkv=8 d=128 bs=16 "
                            "L~U[512,32768]", 128, 32, 8, 128, 512, 32768, True, "fp8", 1004)


@dataclass
class MlaInputs:
    """MLA decode: queries [absorbed latent query ; position query] per head and
    one cache row [latent ; position key] per token (no head axis)."""
    q: torch.Tensor                 # (B, Hq, d_c + d_r) bf16
    kv: torch.Tensor                # contiguous (B, S_cap, d_c + d_r) or pool (nb, bs, d_c + d_r)
    seq_lens: torch.Tensor          # (B,) int32
    block_table: Optional[torch.Tensor]
    block_size: int
    kv_capacity: int
    max_seq_len: int

    def kv_bytes(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum()) * self.kv.shape[-1] * self.kv.element_size()


def make_mla_inputs(B, Hq, d_c, d_r, seed, len_range=None, seq_lens=None, paged=True, block_size=64,
                    s_cap: Optional[int] = None, spare_blocks: int = 0) -> MlaInputs:
    """Seeded MLA decode inputs, drawn like the decode inputs (N(0,1) rounded
    to bf16; lengths uniform and inclusive; a permuted pool with -1 padding and
    NaN in every slot no sequence owns)."""
    g = torch.Generator().manual_seed(seed)
    if seq_lens is None:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)
        max_seq_len = hi
    else:
        lens = torch.tensor(list(seq_lens), dtype=torch.int64)
        max_seq_len = int(lens.max()) if B > 0 else 0
    w = d_c + d_r
    q = _normal(g, (B, Hq, w), "bf16")
    if not paged:
        cap = s_cap if s_cap is not None else max_seq_len
        kv = _normal(g, (B, cap, w), "bf16")
        for b in range(B):
            kv[b, int(lens[b]):] = float("nan")
        return MlaInputs(q, kv, lens.to(torch.int32), None, 0, cap, max_seq_len)
    bs = block_size
    nblk = [(int(L) + bs - 1) // bs for L in lens]
    total = sum(nblk) + spare_blocks
    perm = torch.randperm(total, generator=g)
    mb = max(1, (max_seq_len + bs - 1) // bs)
    table = torch.full((B, mb), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]].to(torch.int32)
        off += nblk[b]
    kv = _normal(g, (total, bs, w), "bf16")
    for b in range(B):
        L = int(lens[b])
        if L % bs:
            kv[int(table[b, nblk[b] - 1]), L % bs:] = float("nan")
    for p in perm[sum(nblk):].tolist():
        kv[p] = float("nan")
    return MlaInputs(q, kv, lens.to(torch.int32), table, bs, total, max_seq_len)


@dataclass(frozen=True)
class MlaWorkload:
    name: str
    B: int
    Hq: int
    d_c: int
    d_r: int
    d_head: int
    len_lo: int
    len_hi: int
    block_size: int
    seed: int

    @property
    def scale(self) -> float:
        """1 / sqrt(d_head + d_r): the score's denominator uses the combined
        width of the content and position parts."""
        return 1.0 / math.sqrt(self.d_head + self.d_r)

    def flops(self, seq_lens) -> int:
        """Per head and cached token: (d_c + d_r) multiply-adds for the score and
        d_c for the weighted sum; 2 flop each."""
        return 2 * self.Hq * (2 * self.d_c + self.d_r) * int(sum(int(L) for L in seq_lens))


def mla_inputs(w: MlaWorkload) -> MlaInputs:
    return make_mla_inputs(w.B, w.Hq, w.d_c, w.d_r, w.seed, len_range=(w.len_lo, w.len_hi), paged=True,
                           block_size=w.block_size)


# DeepSeek-V3-shaped MLA decode batch: 128 heads of width 128 over a 512-wide
# latent plus a 64-wide position key, 128 sequences of 1K-16K cached tokens,
# pages of 64 tokens.
MLA_DECODE = MlaWorkload("MLA decode bf16, B=128 Hq=128 d_c=512 d_r=64 (d_head 128) L~U[1024,16384] bs=64",
                         128, 128, 512, 64, 128, 1024, 16384, 64, 1008)
