/*
 * fa.h — exact softmax attention on AMD Instinct MI355X (gfx950): tiled
 * prefill with the online-softmax recurrence, and single-token decode against
 * a contiguous or paged KV cache.
 *
 * C ABI.  Plain pointers and sizes; no C++ or framework types cross it.
 *
 * Ownership and execution model (all entry points):
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees, or synchronises: work is enqueued on
 *     `stream` (a hipStream_t passed as void*, NULL = the default stream) and
 *     the call returns without waiting for it.
 *   - Tensors are dense and row-major with the head dimension innermost, in the
 *     axis order given with each call; every pointer must be 16-byte aligned.
 *   - Arguments are checked on the host before any HIP call.  A rejected call
 *     returns FA_ERR_INVALID or FA_ERR_UNSUPPORTED and enqueues nothing.  A
 *     failed kernel launch returns FA_ERR_HIP.  No exception crosses the ABI.
 *   - The library is stateless apart from a thread-local error message and is
 *     safe to call from several host threads.
 *   - Outputs are deterministic: the same inputs and launch configuration give
 *     the same bits.  No kernel accumulates a result with atomics; the only
 *     atomics are LDS counters that build a histogram from which a work list
 *     is ordered (the planning step of fa_decode, fa_decode_fp8 and
 *     fa_mla_decode when a sequence spans several splits, and
 *     fa_chunked_prefill over several sequences): the order among equal
 *     lengths may differ between runs, but it decides only which workgroup
 *     computes which part, never a value that is written.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID = 1,     /* an argument breaks the contract below            */
  FA_ERR_UNSUPPORTED = 2, /* valid in principle, not built (e.g. head dim 96) */
  FA_ERR_HIP = 3          /* the HIP runtime reported an error                */
} fa_status;

typedef enum fa_dtype {
  FA_F32 = 0,  /* fp32 in, fp32 out, fp32 arithmetic                       */
  FA_BF16 = 1  /* bf16 in, bf16 out (round to nearest even), fp32 accumulate */
} fa_dtype;

/* Version of this ABI (bumped on any change of a signature or of a workspace size). */
int fa_abi_version(void);

/* Static description of a status code. */
const char* fa_status_string(fa_status s);

/* Detail for the last non-OK status returned on the calling thread ("" if none). */
const char* fa_last_error(void);

/*
 * fa_prefill — attention of every query row against the keys, computed in
 * tiles with the streaming softmax (running max and running sum, earlier
 * partial results rescaled when the max grows), so the Nq x Nk score matrix is
 * never written to memory.
 *
 * Defined by: "KV Cache, Flash Attention and Inference Optimization" (AI
 * Engineering from Scratch, phase 07 lesson 12), section "the tiling trick"
 * (outer loop over query tiles, inner loop over key/value tiles, one write of
 * the output tile); "Module 09: Efficient Attention", sections "The Math:
 * Sharing Keys and Values" (softmax(QK^T/sqrt(d_k))V with query head h reading
 * key/value head floor(h / (Hq/Hkv))) and "FlashAttention: The Compute Wall"
 * (the streaming identity); "Li Hongyi, Machine Learning 2026" notes, lecture
 * "FlashAttention" (the running max/sum recurrence).
 *
 *   q   (B, Hq,  Nq, d)   input dtype
 *   k   (B, Hkv, Nk, d)   input dtype
 *   v   (B, Hkv, Nk, d)   input dtype
 *   o   (B, Hq,  Nq, d)   output, input dtype
 *   lse (B, Hq,  Nq)      fp32 output or NULL: natural log of the sum over
 *                         visible keys of exp(scale * q.k); -inf for a row that
 *                         sees no key
 *   scale                 multiplies q.k before the softmax (finite, > 0;
 *                         1/sqrt(d) for the usual attention)
 *   causal                0: every key visible.  1: key j visible to query i
 *                         iff j <= i + (Nk - Nq), the mask aligned to the
 *                         bottom-right corner so that Nq new queries appended to
 *                         Nk - Nq cached keys see the whole past ("Генерация и
 *                         KV-кэш", section "Три ловушки", item 2)
 *   window                0: no window.  W > 0 (causal only): query i sees
 *                         only keys j > i + (Nk - Nq) - W, i.e. its W most
 *                         recent keys, itself included — the sliding-window
 *                         mask of "Module 09: Efficient Attention", section
 *                         "Attention Mask Gallery"; the work per query is
 *                         then O(W) instead of O(Nk)
 *
 * Contract: B, Nq, Nk >= 0; Hq, Hkv >= 1; Hq % Hkv == 0; d in {64, 128};
 * causal requires Nq <= Nk (otherwise rows with no visible key would exist);
 * window >= 0, and window > 0 requires causal.
 * Nk == 0 (non-causal) yields o = 0 and lse = -inf.  B == 0 or Nq == 0 is a
 * no-op.  q, k, v must not alias o or lse.
 */
int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, int window, float scale, int dtype, void* stream);

/*
 * fa_decode_workspace_bytes — bytes of device workspace fa_decode needs for
 * these sizes (0 when every sequence fits in one split): the splits' partial
 * outputs and log-sum-exps, and the list of (sequence, split) work items that
 * a first small kernel orders longest first.  `window` and `split_tokens` are
 * the values that will be passed to fa_decode (0 = no window / library
 * choice).  Returns 0 for arguments fa_decode would reject.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seq_len, int window,
                                 int split_tokens);

/*
 * fa_decode_split_tokens — tokens per split that fa_decode uses for these
 * sizes when called with split_tokens = 0.
 */
int fa_decode_split_tokens(int B, int Hq, int Hkv, int d, int max_seq_len, int window);

/*
 * fa_decode — one new query per (sequence, query head) against all of that
 * sequence's cached keys and values, the new token's own included (it is
 * already in the cache and counted by seq_lens); no mask.
 *
 * Defined by: "Генерация и KV-кэш" (ai.flicky.cc, stage 4.6 lesson 04),
 * section "KV-кэш для одной головы на NumPy" (decode step = softmax of the new
 * query against every cached key, weighted sum of cached values); "Module 09:
 * Efficient Attention", sections "Code: Cache-Aware Grouped-Query Attention"
 * (the cache stores only Hkv heads) and "Code: A Paged KV Cache from Scratch"
 * (pool of fixed-size blocks, token t of a sequence at
 * (block_table[t / block_size], t % block_size)).
 *
 * The keys of each sequence are cut into splits of `split_tokens`; each split
 * produces a partial (output, log-sum-exp) and a second pass merges the
 * partials of a sequence with weights exp(lse_s - max_s lse_s).
 *
 *   q            (B, Hq, d)              input dtype
 *   k_cache,     contiguous: (B, Hkv, kv_capacity, d), row L_b.. unused
 *   v_cache      paged:      (kv_capacity, block_size, Hkv, d) shared pool
 *   seq_lens     (B) int32, device: cached length L_b of each sequence
 *   block_table  NULL for the contiguous layout, else (B, max_blocks_per_seq)
 *                int32, device: physical block of each logical block; only the
 *                first ceil(L_b / block_size) entries of a row are read
 *   block_size   paged: tokens per block, a power of two in [1, 1024]
 *   max_blocks_per_seq  paged: row length of block_table
 *   kv_capacity  contiguous: S_cap (>= max_seq_len); paged: pool blocks
 *   max_seq_len  host-side upper bound on every L_b (sizes the launch without
 *                reading seq_lens back)
 *   window       0, or W > 0: only the last W cached keys of each sequence
 *                are attended (the sliding window of "Module 09: Efficient
 *                Attention", section "Attention Mask Gallery"); the blocks
 *                before them are not read, so their table entries may be
 *                stale or -1
 *   o            (B, Hq, d) output, input dtype
 *   lse          (B, Hq) fp32 output or NULL
 *   split_tokens 0 = library choice, else tokens per split: a multiple of 256
 *   workspace    device scratch of fa_decode_workspace_bytes(...) bytes, or
 *                NULL when that is 0; contents on entry are ignored
 *
 * Contract: B >= 0; Hq % Hkv == 0; d in {64, 128}; 0 <= L_b <= max_seq_len;
 * for the paged layout every read block id lies in [0, kv_capacity) and
 * max_blocks_per_seq * block_size >= max_seq_len.  L_b == 0 yields o = 0 and
 * lse = -inf.  Device-side violations (an L_b outside [0, max_seq_len], an
 * out-of-range block id) are detected by the kernel: that sequence's rows of
 * o and lse come out NaN and no out-of-range address is read.
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* seq_lens, const int32_t* block_table,
              int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
              void* o, float* lse,
              int B, int Hq, int Hkv, int d, float scale, int dtype,
              int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc — fa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, same kernels and the same results bit for
 * bit as fa_decode with the same split_tokens, but without the workspace: the
 * split partials go to a scratch array that the library holds in each GPU's
 * memory (FA_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends; its address is looked up on the first call on each device).  Nothing
 * is allocated or freed by this call, on the host or the device.
 *
 * Sizes whose partials exceed the array (fa_decode_workspace_bytes(...) >
 * FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_UNSUPPORTED and enqueue
 * nothing.  The array's contents on entry are ignored (every partial that is
 * read was written by the same call) and it keeps the last call's partials.
 * All calls on one GPU share the array: calls that may overlap on one GPU
 * (different streams without ordering between them) race and give undefined
 * results; calls on one stream are ordered and safe.  The stream must belong
 * to the current device.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, const int32_t* block_table,
                      int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
                      void* o, float* lse,
                      int B, int Hq, int Hkv, int d, float scale, int dtype, int split_tokens, void* stream);

/*
 * fa_decode_fp8 — fa_decode against a cache of FP8 codes: one byte per cached
 * number instead of two, so a decode step reads half the bytes.
 *
 * Defined by: fa_decode's passages, plus "Генерация и KV-кэш", section
 * "Сколько весит KV-кэш" (bytes per number: 2 in BF16, 1 in FP8; an FP8 cache
 * is one of the levers on the cache size).  The pages fix nothing more; the
 * library's reading: codes are OCP FP8 E4M3 (bias 7, largest magnitude 448,
 * S.1111.111 = NaN, no infinity) and one fp32 scale per tensor maps a code to
 * the number value(code) * k_scale (keys) or value(code) * v_scale (values).
 *
 *   q, o         (B, Hq, d) bf16
 *   k_cache,     as fa_decode, elements are E4M3 codes (1 byte)
 *   v_cache
 *   k_scale,     finite, > 0
 *   v_scale
 *   everything else as fa_decode (the workspace size is the same:
 *   fa_decode_workspace_bytes)
 */
int fa_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* seq_lens, const int32_t* block_table,
                  int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
                  void* o, float* lse,
                  int B, int Hq, int Hkv, int d, float scale, float k_scale, float v_scale,
                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_kv_append — write the keys and values of n_new new tokens per sequence
 * into a KV cache, at positions L_b - n_new .. L_b - 1 of sequence b (L_b =
 * seq_lens[b], the length AFTER the append).  A pure copy: the cache receives
 * the given bits unchanged.
 *
 * Defined by: "Module 09: Efficient Attention", section "Code: A Paged KV Cache
 * from Scratch" (appending token t writes slot t % block_size of physical block
 * block_table[t / block_size]); "Генерация и KV-кэш", section "KV-кэш для
 * одной головы на NumPy" (each generated token's k and v are appended to the
 * cache before attention reads it).  Claiming blocks is the caller's job: the
 * table must already list the block of every written position.
 *
 *   k_new, v_new (B, Hkv, n_new, d)   input dtype (the layout fa_prefill takes k, v in)
 *   k_cache,     contiguous: (B, Hkv, kv_capacity, d)
 *   v_cache      paged:      (kv_capacity, block_size, Hkv, d) shared pool
 *   seq_lens     (B) int32, device
 *   block_table  NULL (contiguous) or (B, max_blocks_per_seq) int32, device
 *
 * Contract: B, n_new >= 0; Hkv >= 1; d * element size a multiple of 16 bytes;
 * n_new <= L_b <= capacity (contiguous: kv_capacity; paged:
 * max_blocks_per_seq * block_size); block ids read lie in [0, kv_capacity).
 * The new rows must not overlap the cache.  Device-side violations are
 * skipped: a sequence with an L_b outside the contract, or a token whose block
 * id is out of range, is not written, and nothing outside the cache is ever
 * written.  Positions other than the n_new new ones are left untouched.
 */
int fa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* seq_lens, const int32_t* block_table,
                 int block_size, int max_blocks_per_seq, int kv_capacity,
                 int B, int Hkv, int n_new, int d, int dtype, void* stream);

/*
 * fa_kv_append_fp8 — fa_kv_append into an FP8 (E4M3) cache: each bf16 value x
 * of the new rows is stored as the code of x / scale (k_scale for keys,
 * v_scale for values), the quotient formed in fp32 (IEEE division), saturated
 * to +-448 and rounded to the nearest code, ties to the even code; a NaN stays
 * NaN.  The scale convention is the one fa_decode_fp8 reads back.
 *
 *   k_new, v_new (B, Hkv, n_new, d) bf16
 *   k_cache,     (B, Hkv, kv_capacity, d) or (kv_capacity, block_size, Hkv, d)
 *   v_cache      E4M3 codes
 *
 * Contract: as fa_kv_append, with d a multiple of 16 and finite scales > 0.
 */
int fa_kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* seq_lens, const int32_t* block_table,
                     int block_size, int max_blocks_per_seq, int kv_capacity,
                     int B, int Hkv, int n_new, int d, float k_scale, float v_scale, void* stream);

/*
 * fa_mla_decode — multi-head latent attention decode, in the absorbed form:
 * every query head attends one shared cache row per token, [c ; k^R] (the
 * latent, d_c numbers, and the decoupled position key, d_r numbers), with its
 * query [q^lat ; q^R], and outputs the softmax-weighted sum of the latents c
 * (in latent space; the caller applies the value up-projection W^UV).
 *
 * Defined by: "Module 09: Efficient Attention", sections "Multi-head Latent
 * Attention: A Different Lever", "The Math: Compress, Reconstruct, Decouple"
 * (the cache keeps d_c + d_r numbers per token and no head axis; per-head
 * keys are [W^UK c ; k^R]) and "Why RoPE Has To Be Decoupled" (the content
 * up-projections absorb into the query: q^C . W^UK c = (W^UK^T q^C) . c).
 * The caller forms q^lat = W^UK^T q^C and applies RoPE to q^R and k^R; scale
 * is 1 / sqrt(d_head + d_r) for the page's model ("Common Pitfalls" item 7).
 *
 *   q            (B, Hq, d_c + d_r) bf16: [q^lat ; q^R] per head
 *   kv_cache     contiguous: (B, kv_capacity, d_c + d_r); paged:
 *                (kv_capacity, block_size, d_c + d_r) pool, bf16 rows [c ; k^R]
 *   seq_lens, block_table, block_size, max_blocks_per_seq, max_seq_len: as
 *                fa_decode (one shared row per token instead of Hkv heads)
 *   o            (B, Hq, d_c) bf16 output
 *   lse          (B, Hq) fp32 output or NULL
 *   split_tokens 0 = library choice (fa_mla_decode_split_tokens), else a
 *                multiple of 32: a sequence of L tokens is cut into
 *                ceil(L / split_tokens) parts of equal length (rounded up to
 *                32 tokens), whose partials are merged
 *   workspace    fa_mla_decode_workspace_bytes(...) bytes (NULL if 0)
 *
 * Contract: d_c = 512 and d_r = 64 (the shape built); 0 <= L_b <= max_seq_len;
 * block ids read in [0, kv_capacity).  Device-side violations give NaN rows
 * and no out-of-range read, as for fa_decode.
 */
int fa_mla_decode(const void* q, const void* kv_cache, const int32_t* seq_lens, const int32_t* block_table,
                  int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len,
                  void* o, float* lse, int B, int Hq, int d_c, int d_r, float scale,
                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* Tokens per split fa_mla_decode uses when called with split_tokens = 0 (0 for rejected sizes). */
int fa_mla_decode_split_tokens(int B, int Hq, int d_c, int d_r, int max_seq_len);

/* Workspace bytes fa_mla_decode needs (0 when every sequence fits in one split or the sizes are rejected):
 * the split partials (B x Hq x splits x d_c bf16, then their fp32 log-sum-exps)
 * and a work list (1 + B x splits int32) that orders the splits longest first. */
size_t fa_mla_decode_workspace_bytes(int B, int Hq, int d_c, int d_r, int max_seq_len, int split_tokens);

/*
 * fa_chunked_prefill — attention of the Nq newest tokens of each sequence
 * against that sequence's whole KV cache (its own new keys included, appended
 * beforehand, e.g. by fa_kv_append): the prefill of one chunk of a long prompt,
 * or of a prompt that extends a cached prefix.  Query i of sequence b is the
 * token at position L_b - Nq + i and, when causal, sees keys
 * j <= L_b - Nq + i: the causal mask aligned to the bottom-right corner
 * ("Генерация и KV-кэш", section "Три ловушки", item 2).  Nq = 1 is a decode
 * step (fa_decode computes the same thing with a split-K launch).
 *
 * Defined by: the same passages as fa_prefill (tiled exact attention with the
 * streaming softmax) with keys read through the cache layout of fa_decode
 * ("Module 09: Efficient Attention", section "Code: A Paged KV Cache from
 * Scratch").
 *
 *   q            (B, Hq, Nq, d)          input dtype
 *   k_cache,     contiguous: (B, Hkv, kv_capacity, d)
 *   v_cache      paged:      (kv_capacity, block_size, Hkv, d) shared pool
 *   seq_lens     (B) int32, device: cached length L_b, the Nq new tokens included
 *   block_table  NULL (contiguous) or (B, max_blocks_per_seq) int32, device
 *   max_seq_len  host-side upper bound on every L_b
 *   o            (B, Hq, Nq, d) output, input dtype
 *   lse          (B, Hq, Nq) fp32 output or NULL (as for fa_prefill)
 *   causal       1 for a prompt chunk; 0 lets every query see all L_b keys
 *   window       as fa_prefill (positions counted in the whole sequence); the
 *                blocks before the first window of the chunk are not read
 *
 * Contract: as fa_prefill for B, heads, d, scale, window; 0 <= L_b <= max_seq_len and,
 * when causal, L_b >= Nq; contiguous kv_capacity >= max_seq_len; paged:
 * block_size a power of two in [1, 1024], max_blocks_per_seq * block_size >=
 * max_seq_len and every block id read in [0, kv_capacity).  Device-side
 * violations (an L_b outside that range, an out-of-range block id) are
 * detected by the kernel: the affected rows of o and lse come out NaN and no
 * out-of-range address is read.
 */
int fa_chunked_prefill(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len,
                       void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int d,
                       int causal, int window, float scale, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
