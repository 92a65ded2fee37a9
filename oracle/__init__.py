"""CPU fp64 oracle for exact softmax attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls anything here, and this package imports
nothing from the product: the two share no code.  Inputs reach both sides from
the seeded generators, which hold no attention arithmetic.

Modules:
  attention  the plain definition: materialise the scores, two-pass softmax,
             GQA head mapping, bottom-right causal mask and sliding window,
             contiguous and paged KV-cache reads (prefill and decode).
  online     the pages' streaming recurrence (running max and sum, rescaling of
             earlier partials) and the merge of two partial states; used to pin
             the definition, never to produce expected values for kernels.
  kv_bytes   the KV-cache size formula.
  paged      the paged pool: free-list block allocation, token append through
             the block table, prefix sharing, and chunked prefill (the newest
             Nq tokens of each sequence against its whole cache).
  mla        multi-head latent attention decode: the latent-space form the
             kernel computes, and the head-by-head form built from the page's
             equations (the absorption identity pins one against the other).
  fp8        FP8 (E4M3) caches: the code -> value table from the bit layout,
             round-to-nearest-even quantisation with saturation, per-tensor
             scales, decode against an FP8 cache, quantising append.

Every function cites the passage it follows by page title and section.  All
functions are pinned by tests that check them against values the pages print,
closed forms, special cases and brute force (no function is "parity unpinned").
"""
from .attention import (kv_head_of, causal_key_limit, window_key_start, attention_rows, prefill,
                        prefill_rows, paged_gather, decode_contiguous, decode_paged)
from .online import online_softmax_stats, online_attention_row, merge_partials
from .kv_bytes import kv_cache_bytes, kv_bytes_per_token
from .paged import (BlockAllocator, PagedSequence, append_token, share_prefix, append_batch,
                    append_batch_contiguous, chunked_prefill)
from .fp8 import e4m3_value, decode_codes, quantize_e4m3, decode_fp8, append_fp8
from .mla import (mla_cache_numbers, mha_cache_numbers, equivalent_gqa_groups, absorb_query,
                  mla_decode_latent, mla_decode_explicit, latent_to_head)

__all__ = [
    "kv_head_of", "causal_key_limit", "window_key_start", "attention_rows", "prefill", "prefill_rows",
    "paged_gather", "decode_contiguous", "decode_paged",
    "online_softmax_stats", "online_attention_row", "merge_partials",
    "kv_cache_bytes", "kv_bytes_per_token",
    "BlockAllocator", "PagedSequence", "append_token", "share_prefix", "append_batch",
    "append_batch_contiguous", "chunked_prefill",
    "e4m3_value", "decode_codes", "quantize_e4m3", "decode_fp8", "append_fp8",
    "mla_cache_numbers", "mha_cache_numbers", "equivalent_gqa_groups", "absorb_query",
    "mla_decode_latent", "mla_decode_explicit", "latent_to_head",
]
