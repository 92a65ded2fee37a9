"""Multi-head latent attention (MLA) decode on the CPU (test infrastructure only).

What is computed, and where the page says so ("Module 09: Efficient
Attention", sections "Multi-head Latent Attention: A Different Lever", "The
Math: Compress, Reconstruct, Decouple", "Why RoPE Has To Be Decoupled" and
"Common Pitfalls" items 6-7):

* the cache keeps, per token, the latent c_j (d_c numbers) and one decoupled
  position key k^R_j (d_r numbers, already rotated) shared by all heads;
* head i reconstructs its content key and value from the latent,
  k^C_{j,i} = W^UK_i c_j and v_{j,i} = W^UV_i c_j, and its key is the
  concatenation [k^C_{j,i} ; k^R_j]; its query is [q^C_i ; q^R_i];
* the score is q_i . k_{j,i} / sqrt(d_head + d_r) — the combined width
  (pitfall 7);
* absorption: q^C_i . (W^UK_i c_j) = (W^UK_i^T q^C_i) . c_j, so with the
  absorbed query q^lat_i = W^UK_i^T q^C_i a head attends the cached latent
  directly, and because the value is linear in c_j the head's output is
  W^UV_i applied to the softmax-weighted sum of latents.

``mla_decode_latent`` is what the decode kernel computes: every head attends
the cached rows [c_j ; k^R_j] with its query [q^lat_i ; q^R_i], the values
being the latents c_j (one shared "KV head" with key width d_c + d_r and value
width d_c).  ``mla_decode_explicit`` builds the per-head keys and values from
the equations instead; the two agree (the absorption identity), which pins the
first against the page's definition.

Reading taken: a cache row holds [c_j ; k^R_j] contiguously (d_c + d_r
numbers), the layout the kernels read; the page's cache keeps the same
numbers in two tensors.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _i64, attention_rows, paged_gather


def mla_cache_numbers(d_c: int, d_r: int, layers: int = 1) -> int:
    """Numbers cached per token: d_c + d_r per layer, no head factor."""
    return layers * (d_c + d_r)


def mha_cache_numbers(heads: int, head_dim: int, layers: int = 1) -> int:
    """Numbers an MHA cache keeps per token: a key and a value per head."""
    return layers * 2 * heads * head_dim


def equivalent_gqa_groups(d_c: int, d_r: int, head_dim: int) -> float:
    """How many GQA KV heads cache as much as one MLA token row."""
    return (d_c + d_r) / (2 * head_dim)


def absorb_query(q_c, w_uk):
    """q^lat_i = W^UK_i^T q^C_i.  q_c (B, H, d_head), w_uk (H, d_head, d_c)."""
    return np.einsum("bhe,hec->bhc", _f64(q_c), _f64(w_uk))


def _rows(kv, b, L, block_table, block_size):
    """The L cached rows of sequence b (contiguous (B, S_cap, w) or paged
    (num_blocks, block_size, w))."""
    if block_table is None:
        return _f64(kv[b, :L])
    return paged_gather(kv[:, :, None, :], _i64(block_table)[b], L, 0, block_size)


def mla_decode_latent(q, kv, seq_lens, scale: float, d_c: int, block_table=None, block_size: int = 0,
                      heads=None):
    """q (B, H, d_c + d_r): [absorbed content query ; position query] per head;
    kv: cache rows [c_j ; k^R_j].  Returns O (B, H, d_c) — each head's output in
    latent space — and LSE (B, H); rows not computed (``heads`` restricts to a
    list of (b, h)) are left NaN."""
    B, H, w = q.shape
    lens = _i64(seq_lens)
    O = np.full((B, H, d_c), np.nan)
    lse = np.full((B, H), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    # every head of a sequence attends the same cache rows: one score matrix
    # per sequence, one row per requested head
    by_seq = {}
    for b, h in todo:
        by_seq.setdefault(b, []).append(h)
    for b, hs in by_seq.items():
        K = _rows(kv, b, int(lens[b]), block_table, block_size)
        o, l = attention_rows(_f64(q[b, hs]), K, K[:, :d_c], scale)
        O[b, hs], lse[b, hs] = o, l
    return O, lse


def mla_decode_explicit(q_c, q_r, w_uk, w_uv, latent, k_rope, seq_lens, scale: float):
    """MLA decode built from the page's equations, per head.

    q_c (B, H, d_head), q_r (B, H, d_r); w_uk, w_uv (H, d_head, d_c); latent
    (B, S, d_c) and k_rope (B, S, d_r) contiguous caches.  Returns the head
    outputs (B, H, d_head) and LSE (B, H)."""
    q_c, q_r, w_uk, w_uv = _f64(q_c), _f64(q_r), _f64(w_uk), _f64(w_uv)
    latent, k_rope = _f64(latent), _f64(k_rope)
    B, H, d_head = q_c.shape
    lens = _i64(seq_lens)
    O = np.zeros((B, H, d_head))
    lse = np.zeros((B, H))
    for b in range(B):
        L = int(lens[b])
        c = latent[b, :L]
        for h in range(H):
            k_c = c @ w_uk[h].T                         # (L, d_head): W^UK_h c_j
            v = c @ w_uv[h].T                           # (L, d_head): W^UV_h c_j
            K = np.concatenate([k_c, k_rope[b, :L]], axis=1)
            qh = np.concatenate([q_c[b, h], q_r[b, h]])[None]
            o, l = attention_rows(qh, K, v, scale)
            O[b, h], lse[b, h] = o[0], l[0]
    return O, lse


def latent_to_head(o_lat, w_uv):
    """A head's output from its latent-space output: W^UV_i o^lat_i."""
    return np.einsum("hec,bhc->bhe", _f64(w_uv), _f64(o_lat))
