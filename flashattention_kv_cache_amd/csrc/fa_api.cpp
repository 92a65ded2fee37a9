// Host side of the C ABI declared in include/fa.h: argument checks (all done
// before any HIP call), launch planning, and error reporting.
#include "../../include/fa.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fa_internal.h"

namespace {

thread_local char g_err[256] = "";

int fail(fa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(fa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

int ok() {
  g_err[0] = '\0';
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Tokens per decode split when the caller leaves the choice to the library:
// about 12288 splits over (sequence, KV head group) pairs if every sequence
// had max_seq_len tokens, rounded up to a multiple of 512 (256 below 1024)
// and kept within [1024, 4096] — [256, 4096] when there are fewer than 256
// pairs.  Longer splits amortise each workgroup's fixed cost (block
// table prologue, final reductions); shorter ones shrink the tail of the last
// dispatch round.  Measured on MI355X: 3072 for 128 paged sequences of up to
// 32768 tokens, 1024 for 64 contiguous sequences of up to 8192.
int choose_split_tokens(int B, int Hq, int Hkv, int max_seq_len) {
  const int n_rep = Hq / Hkv;
  const int qh = n_rep % 8 == 0 ? 8 : n_rep % 4 == 0 ? 4 : n_rep % 2 == 0 ? 2 : 1;
  const double pairs = (double)B * Hkv * (n_rep / qh);
  // at least four workgroups per CU and short spans (a sliding window): one
  // split per pair, no merge (measured on MI355X: 6.6% faster than 1024-token
  // splits for 128 sequences x 8 KV heads with a 4096-token window)
  if (pairs >= 1024 && max_seq_len <= 4096) return max(256, (max_seq_len + 255) / 256 * 256);
  // Splits run longest first, so a long split no longer leaves the last
  // workgroups' slots idle, and fewer, longer splits save per-workgroup
  // start-up and merge work.  Aim at about three rounds of 512 workgroups
  // (two per CU) with sequences averaging half of max_seq_len: measured on
  // MI355X over 1024..24576-token splits, this lands within 1% of the best
  // split for the paged B = 128 batch (bf16 and FP8) and within 2% for the
  // contiguous B = 64 one.
  const double want = pairs * (double)max_seq_len / 3072.0;
  // with few pairs, short splits are what fills the GPU
  const long long lo = pairs >= 256 ? 1024 : 256, step = want >= 1024 ? 512 : 256;
  long long st = ((long long)want + step - 1) / step * step;
  if (st < lo) st = lo;
  if (st > 16384) st = 16384;
  return (int)st;
}

int check_decode_sizes(int B, int Hq, int Hkv, int d, int max_seq_len, int split_tokens) {
  if (B < 0 || Hq < 1 || Hkv < 1 || max_seq_len < 0)
    return fail(FA_ERR_INVALID, "B=%d Hq=%d Hkv=%d max_seq_len=%d: need B >= 0, heads >= 1, max_seq_len >= 0",
                B, Hq, Hkv, max_seq_len);
  if (Hq % Hkv) return fail(FA_ERR_INVALID, "num_kv_heads (%d) must divide num_heads (%d)", Hkv, Hq);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d not built (64 or 128)", d);
  if (split_tokens < 0 || split_tokens % 256)
    return fail(FA_ERR_INVALID, "split_tokens %d must be 0 or a positive multiple of 256", split_tokens);
  return FA_OK;
}

// Shape of a KV cache as the cached-key entry points take it (contiguous or paged).
int check_cache_layout(const int32_t* block_table, int block_size, int max_blocks_per_seq, int kv_capacity,
                       int max_seq_len) {
  if (max_seq_len < 0) return fail(FA_ERR_INVALID, "max_seq_len %d must be >= 0", max_seq_len);
  if (block_table) {
    if (!is_pow2(block_size) || block_size > 1024)
      return fail(FA_ERR_INVALID, "block_size %d must be a power of two in [1, 1024]", block_size);
    if (kv_capacity < 1) return fail(FA_ERR_INVALID, "paged pool must hold at least one block");
    if (max_blocks_per_seq < 1) return fail(FA_ERR_INVALID, "max_blocks_per_seq must be >= 1");
    if ((long long)max_blocks_per_seq * block_size < max_seq_len)
      return fail(FA_ERR_INVALID, "max_blocks_per_seq (%d) * block_size (%d) < max_seq_len (%d)",
                  max_blocks_per_seq, block_size, max_seq_len);
    if (reinterpret_cast<uintptr_t>(block_table) & 3u) return fail(FA_ERR_INVALID, "block_table must be 4-byte aligned");
  } else {
    if (kv_capacity < max_seq_len || kv_capacity < 1)
      return fail(FA_ERR_INVALID, "contiguous cache capacity %d must be >= max(1, max_seq_len %d)", kv_capacity,
                  max_seq_len);
  }
  return FA_OK;
}

int check_window(int window, int causal) {
  if (window < 0) return fail(FA_ERR_INVALID, "window %d must be >= 0 (0 = no window)", window);
  if (window > 0 && !causal) return fail(FA_ERR_INVALID, "a sliding window needs causal attention");
  return FA_OK;
}

// Longest key range a decode query can see: the sliding window caps it.
int decode_span(int max_seq_len, int window) {
  return window > 0 && window < max_seq_len ? window : max_seq_len;
}

// MLA decode: one workgroup fills a CU, and the splits run longest first, so
// the split length aims at just under two rounds of workgroups on the 256
// CUs.  The host knows only max_seq_len: the mean length is taken as half of
// it, so a launch has about groups * (max_seq_len / 2 / st + 1/2) work items;
// st solves that for 1.9 x 256.  Multiples of 256, within [1024, 16384].
// Measured on MI355X, 128 sequences of up to 16384 tokens with 128 heads:
// 2560 tokens (0.473 ms); 2304 (a third, nearly empty round) 0.571 ms, 3072
// 0.485 ms.
int choose_mla_split_tokens(int B, int Hq, int max_seq_len) {
  const double groups = (double)B * ((Hq + 127) / 128);  // workgroups per split position
  const double room = 1.9 * 256 - 0.5 * groups;
  long long st = room > 0 ? (long long)(groups * 0.5 * max_seq_len / room) : (long long)max_seq_len;
  st = (st + 255) / 256 * 256;
  if (st < 1024) st = 1024;
  if (st > 16384) st = 16384;
  return (int)st;
}

int check_mla_sizes(int B, int Hq, int d_c, int d_r, int max_seq_len, int split_tokens) {
  if (B < 0 || Hq < 1 || max_seq_len < 0)
    return fail(FA_ERR_INVALID, "B=%d Hq=%d max_seq_len=%d: need B >= 0, Hq >= 1, max_seq_len >= 0", B, Hq,
                max_seq_len);
  if (d_c != 512 || d_r != 64)
    return fail(FA_ERR_UNSUPPORTED, "latent width %d + position key %d not built (512 + 64)", d_c, d_r);
  if (split_tokens < 0 || split_tokens % 32)
    return fail(FA_ERR_INVALID, "split_tokens %d must be 0 or a positive multiple of 32", split_tokens);
  return FA_OK;
}

int max_splits_for(int max_seq_len, int split_tokens) {
  return max_seq_len <= split_tokens ? 1 : (max_seq_len + split_tokens - 1) / split_tokens;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 7; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fa_last_error(void) { return g_err; }

int fa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int d,
               int causal, int window, float scale, int dtype, void* stream) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1)
    return fail(FA_ERR_INVALID, "B=%d Hq=%d Hkv=%d Nq=%d Nk=%d: sizes must be >= 0 and heads >= 1", B, Hq, Hkv, Nq, Nk);
  if (Hq % Hkv) return fail(FA_ERR_INVALID, "num_kv_heads (%d) must divide num_heads (%d)", Hkv, Hq);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d not built (64 or 128)", d);
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID, "causal must be 0 or 1, got %d", causal);
  if (causal && Nq > Nk)
    return fail(FA_ERR_INVALID, "causal attention with Nq=%d > Nk=%d would leave rows with no visible key", Nq, Nk);
  if (check_window(window, causal) != FA_OK) return FA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite and > 0");
  if (B == 0 || Nq == 0) return ok();
  if (!q || !o || (Nk > 0 && (!k || !v))) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  const long long rows = (long long)B * Hq * Nq;
  if (rows * d >= (1ll << 40)) return fail(FA_ERR_UNSUPPORTED, "problem too large");

  fa::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = Nk; a.d = d;
  a.causal = causal; a.window = window; a.scale = scale;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == FA_BF16 ? fa::launch_prefill_bf16(a, st) : fa::launch_prefill_f32(a, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fa_chunked_prefill(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len,
                       void* o, float* lse,
                       int B, int Hq, int Hkv, int Nq, int d,
                       int causal, int window, float scale, int dtype, void* stream) {
  if (B < 0 || Nq < 0 || Hq < 1 || Hkv < 1)
    return fail(FA_ERR_INVALID, "B=%d Hq=%d Hkv=%d Nq=%d: sizes must be >= 0 and heads >= 1", B, Hq, Hkv, Nq);
  if (Hq % Hkv) return fail(FA_ERR_INVALID, "num_kv_heads (%d) must divide num_heads (%d)", Hkv, Hq);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dim %d not built (64 or 128)", d);
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID, "causal must be 0 or 1, got %d", causal);
  if (check_window(window, causal) != FA_OK) return FA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite and > 0");
  int st0 = check_cache_layout(block_table, block_size, max_blocks_per_seq, kv_capacity, max_seq_len);
  if (st0 != FA_OK) return st0;
  if (causal && Nq > max_seq_len)
    return fail(FA_ERR_INVALID, "causal chunk of Nq=%d queries exceeds max_seq_len=%d", Nq, max_seq_len);
  if (B == 0 || Nq == 0) return ok();
  if (!q || !k_cache || !v_cache || !seq_lens || !o) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FA_ERR_INVALID, "seq_lens must be 4-byte aligned");
  const long long rows = (long long)B * Hq * Nq;
  if (rows * d >= (1ll << 40)) return fail(FA_ERR_UNSUPPORTED, "problem too large");

  fa::PrefillArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nk = 0; a.d = d;
  a.causal = causal; a.window = window; a.scale = scale;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.block_size = block_table ? block_size : 0;
  a.log2_block_size = block_table ? ilog2(block_size) : 0;
  a.max_blocks_per_seq = block_table ? max_blocks_per_seq : 0;
  a.kv_capacity = kv_capacity;
  a.max_seq_len = max_seq_len;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == FA_BF16 ? fa::launch_prefill_bf16(a, st) : fa::launch_prefill_f32(a, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* seq_lens, const int32_t* block_table,
                 int block_size, int max_blocks_per_seq, int kv_capacity,
                 int B, int Hkv, int n_new, int d, int dtype, void* stream) {
  if (B < 0 || Hkv < 1 || n_new < 0 || d < 1)
    return fail(FA_ERR_INVALID, "B=%d Hkv=%d n_new=%d d=%d: need B, n_new >= 0 and Hkv, d >= 1", B, Hkv, n_new, d);
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  const int es = dtype == FA_BF16 ? 2 : 4;
  if ((d * es) % 16) return fail(FA_ERR_UNSUPPORTED, "a (token, head) row of %d bytes is not a multiple of 16", d * es);
  int st0 = check_cache_layout(block_table, block_size, max_blocks_per_seq, kv_capacity, 0);
  if (st0 != FA_OK) return st0;
  if (B == 0 || n_new == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FA_ERR_INVALID, "seq_lens must be 4-byte aligned");
  if ((long long)B * Hkv > 65535) return fail(FA_ERR_UNSUPPORTED, "B * Hkv must be <= 65535");
  if ((long long)n_new * (d * es / 16) > 0x7fffffffll) return fail(FA_ERR_UNSUPPORTED, "n_new too large");

  fa::AppendArgs a{};
  a.k_new = k_new; a.v_new = v_new; a.k = k_cache; a.v = v_cache;
  a.seq_lens = seq_lens; a.block_table = block_table;
  a.block_size = block_table ? block_size : 0;
  a.log2_block_size = block_table ? ilog2(block_size) : 0;
  a.max_blocks_per_seq = block_table ? max_blocks_per_seq : 0;
  a.kv_capacity = kv_capacity;
  a.B = B; a.Hkv = Hkv; a.n_new = n_new; a.row_chunks = d * es / 16;
  hipError_t e = fa::launch_kv_append(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fa_decode_split_tokens(int B, int Hq, int Hkv, int d, int max_seq_len, int window) {
  if (check_decode_sizes(B, Hq, Hkv, d, max_seq_len, 0) != FA_OK || window < 0) return 0;
  return choose_split_tokens(B, Hq, Hkv, decode_span(max_seq_len, window));
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_seq_len, int window, int split_tokens) {
  if (check_decode_sizes(B, Hq, Hkv, d, max_seq_len, split_tokens) != FA_OK || window < 0) return 0;
  const int span = decode_span(max_seq_len, window);
  const int st = split_tokens ? split_tokens : choose_split_tokens(B, Hq, Hkv, span);
  const int ns = max_splits_for(span, st);
  if (ns <= 1) return 0;
  const size_t slots = (size_t)B * Hq * ns;
  // partial outputs (d floats per slot), partial LSEs, then the work list of
  // the (sequence, split) items, each 256-byte aligned
  const size_t o_bytes = (slots * d * sizeof(float) + 255) & ~(size_t)255;
  const size_t l_bytes = (slots * sizeof(float) + 255) & ~(size_t)255;
  const size_t p_bytes = ((1 + (size_t)B * ns) * sizeof(int32_t) + 255) & ~(size_t)255;
  return o_bytes + l_bytes + p_bytes;
}

}  // extern "C"

namespace {

// Split partials of fa_decode_noalloc: one array per GPU, in the code object's
// device memory, so that call allocates nothing.  In host code `scratch` names
// a host-side stand-in; its device address comes from hipGetSymbolAddress,
// looked up once per device (with that device current) and kept here.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FA_ERR_HIP, "scratch address lookup on device %d failed: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// fa_decode and fa_decode_fp8 share everything but the cache element type.
// static_scratch: the split partials go to this device's scratch array
// (workspace and workspace_bytes are ignored).
int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens, const int32_t* block_table,
                int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
                void* o, float* lse,
                int B, int Hq, int Hkv, int d, float scale, fa::KvType kv, float k_scale, float v_scale,
                int split_tokens, void* workspace, size_t workspace_bytes, void* stream,
                bool static_scratch = false) {
  int st0 = check_decode_sizes(B, Hq, Hkv, d, max_seq_len, split_tokens);
  if (st0 != FA_OK) return st0;
  if (check_window(window, 1) != FA_OK) return FA_ERR_INVALID;
  if (!(scale > 0.f) || !isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite and > 0");
  if (!(k_scale > 0.f) || !isfinite(k_scale) || !(v_scale > 0.f) || !isfinite(v_scale))
    return fail(FA_ERR_INVALID, "k_scale and v_scale must be finite and > 0");
  const bool paged = block_table != nullptr;
  if (paged) {
    if (!is_pow2(block_size) || block_size > 1024)
      return fail(FA_ERR_INVALID, "block_size %d must be a power of two in [1, 1024]", block_size);
    if (kv_capacity < 1) return fail(FA_ERR_INVALID, "paged pool must hold at least one block");
    if ((long long)max_blocks_per_seq * block_size < max_seq_len)
      return fail(FA_ERR_INVALID, "max_blocks_per_seq (%d) * block_size (%d) < max_seq_len (%d)",
                  max_blocks_per_seq, block_size, max_seq_len);
  } else {
    if (kv_capacity < max_seq_len)
      return fail(FA_ERR_INVALID, "contiguous cache capacity %d < max_seq_len %d", kv_capacity, max_seq_len);
  }
  if (B == 0) return ok();
  if (!q || !k_cache || !v_cache || !seq_lens || !o) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return fail(FA_ERR_INVALID, "seq_lens and block_table must be 4-byte aligned");
  if (kv_capacity < 1) return fail(FA_ERR_INVALID, "KV capacity must be >= 1");

  const int span = decode_span(max_seq_len, window);
  const int stoks = split_tokens ? split_tokens : choose_split_tokens(B, Hq, Hkv, span);
  const int ns = max_splits_for(span, stoks);
  const size_t need = fa_decode_workspace_bytes(B, Hq, Hkv, d, max_seq_len, window, split_tokens);
  if (static_scratch) {
    if (need > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES)
      return fail(FA_ERR_UNSUPPORTED, "split partials need %zu bytes, more than the %zu-byte scratch array",
                  need, (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    workspace_bytes = 0;
  } else if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(FA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  if (B > 65535 || Hq > 65535 || ns > 65535 || (long long)Hq * B * ns > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "grid too large (B, Hq and the number of splits must be <= 65535, "
                "and Hq * B * splits < 2^31)");
  if (static_scratch && need > 0) {  // every argument checked: now the (first-call) address lookup
    const int sc = current_scratch(&workspace);
    if (sc != FA_OK) return sc;
  }

  fa::DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.seq_lens = seq_lens; a.block_table = block_table;
  a.block_size = paged ? block_size : 0;
  a.log2_block_size = paged ? ilog2(block_size) : 0;
  a.max_blocks_per_seq = paged ? max_blocks_per_seq : 0;
  a.kv_capacity = kv_capacity; a.max_seq_len = max_seq_len; a.window = window;
  a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.scale = scale;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.split_tokens = stoks; a.max_splits = ns;
  if (ns > 1) {
    const size_t slots = (size_t)B * Hq * ns;
    const size_t o_bytes = (slots * d * sizeof(float) + 255) & ~(size_t)255;
    const size_t l_bytes = (slots * sizeof(float) + 255) & ~(size_t)255;
    a.ws_o = reinterpret_cast<float*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + o_bytes);
    a.plan = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + o_bytes + l_bytes);
  }
  hipError_t e = fa::launch_decode(a, kv, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* seq_lens, const int32_t* block_table,
              int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
              void* o, float* lse,
              int B, int Hq, int Hkv, int d, float scale, int dtype,
              int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  return decode_impl(q, k_cache, v_cache, seq_lens, block_table, block_size, max_blocks_per_seq, kv_capacity,
                     max_seq_len, window, o, lse, B, Hq, Hkv, d, scale,
                     dtype == FA_BF16 ? fa::KvType::BF16 : fa::KvType::F32, 1.f, 1.f,
                     split_tokens, workspace, workspace_bytes, stream);
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, const int32_t* block_table,
                      int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
                      void* o, float* lse,
                      int B, int Hq, int Hkv, int d, float scale, int dtype, int split_tokens, void* stream) {
  if (dtype != FA_F32 && dtype != FA_BF16) return fail(FA_ERR_INVALID, "unknown dtype %d", dtype);
  return decode_impl(q, k_cache, v_cache, seq_lens, block_table, block_size, max_blocks_per_seq, kv_capacity,
                     max_seq_len, window, o, lse, B, Hq, Hkv, d, scale,
                     dtype == FA_BF16 ? fa::KvType::BF16 : fa::KvType::F32, 1.f, 1.f,
                     split_tokens, nullptr, 0, stream, /*static_scratch=*/true);
}

int fa_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* seq_lens, const int32_t* block_table,
                  int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len, int window,
                  void* o, float* lse,
                  int B, int Hq, int Hkv, int d, float scale, float k_scale, float v_scale,
                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_cache, v_cache, seq_lens, block_table, block_size, max_blocks_per_seq, kv_capacity,
                     max_seq_len, window, o, lse, B, Hq, Hkv, d, scale, fa::KvType::FP8, k_scale, v_scale,
                     split_tokens, workspace, workspace_bytes, stream);
}

int fa_mla_decode_split_tokens(int B, int Hq, int d_c, int d_r, int max_seq_len) {
  if (check_mla_sizes(B, Hq, d_c, d_r, max_seq_len, 0) != FA_OK) return 0;
  return choose_mla_split_tokens(B, Hq, max_seq_len);
}

size_t fa_mla_decode_workspace_bytes(int B, int Hq, int d_c, int d_r, int max_seq_len, int split_tokens) {
  if (check_mla_sizes(B, Hq, d_c, d_r, max_seq_len, split_tokens) != FA_OK) return 0;
  const int st = split_tokens ? split_tokens : choose_mla_split_tokens(B, Hq, max_seq_len);
  const int ns = max_splits_for(max_seq_len, st);
  if (ns <= 1) return 0;
  const size_t slots = (size_t)B * Hq * ns;
  // bf16 partial outputs (they are normalised, and the output itself is bf16),
  // fp32 log-sum-exps, then the work list
  const size_t o_bytes = (slots * d_c * sizeof(uint16_t) + 255) & ~(size_t)255;
  const size_t l_bytes = (slots * sizeof(float) + 255) & ~(size_t)255;
  const size_t p_bytes = ((1 + (size_t)B * ns) * sizeof(int32_t) + 255) & ~(size_t)255;
  return o_bytes + l_bytes + p_bytes;
}

int fa_mla_decode(const void* q, const void* kv_cache, const int32_t* seq_lens, const int32_t* block_table,
                  int block_size, int max_blocks_per_seq, int kv_capacity, int max_seq_len,
                  void* o, float* lse, int B, int Hq, int d_c, int d_r, float scale,
                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  int st0 = check_mla_sizes(B, Hq, d_c, d_r, max_seq_len, split_tokens);
  if (st0 != FA_OK) return st0;
  if (!(scale > 0.f) || !isfinite(scale)) return fail(FA_ERR_INVALID, "scale must be finite and > 0");
  st0 = check_cache_layout(block_table, block_size, max_blocks_per_seq, kv_capacity, max_seq_len);
  if (st0 != FA_OK) return st0;
  if (B == 0) return ok();
  if (!q || !kv_cache || !seq_lens || !o) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(o) || !aligned16(lse))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FA_ERR_INVALID, "seq_lens must be 4-byte aligned");
  const int stoks = split_tokens ? split_tokens : choose_mla_split_tokens(B, Hq, max_seq_len);
  const int ns = max_splits_for(max_seq_len, stoks);
  const size_t need = fa_mla_decode_workspace_bytes(B, Hq, d_c, d_r, max_seq_len, split_tokens);
  if (need > 0) {
    if (!workspace) return fail(FA_ERR_INVALID, "workspace of %zu bytes required", need);
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(FA_ERR_INVALID, "workspace must be 256-byte aligned");
  }
  if (B > 65535 || (long long)B * ns >= 0x7fffffff || (Hq + 127) / 128 > 65535)
    return fail(FA_ERR_UNSUPPORTED, "grid too large (B <= 65535)");

  fa::MlaArgs a{};
  a.q = q; a.kv = kv_cache; a.seq_lens = seq_lens; a.block_table = block_table;
  a.block_size = block_table ? block_size : 0;
  a.log2_block_size = block_table ? ilog2(block_size) : 0;
  a.max_blocks_per_seq = block_table ? max_blocks_per_seq : 0;
  a.kv_capacity = kv_capacity; a.max_seq_len = max_seq_len;
  a.o = o; a.lse = lse; a.B = B; a.Hq = Hq; a.scale = scale;
  a.split_tokens = stoks; a.max_splits = ns;
  if (ns > 1) {
    const size_t slots = (size_t)B * Hq * ns;
    const size_t o_bytes = (slots * d_c * sizeof(uint16_t) + 255) & ~(size_t)255;
    const size_t l_bytes = (slots * sizeof(float) + 255) & ~(size_t)255;
    a.ws_o = reinterpret_cast<uint16_t*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + o_bytes);
    a.plan = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + o_bytes + l_bytes);
  }
  hipError_t e = fa::launch_mla_decode(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fa_kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* seq_lens, const int32_t* block_table,
                     int block_size, int max_blocks_per_seq, int kv_capacity,
                     int B, int Hkv, int n_new, int d, float k_scale, float v_scale, void* stream) {
  if (B < 0 || Hkv < 1 || n_new < 0 || d < 1)
    return fail(FA_ERR_INVALID, "B=%d Hkv=%d n_new=%d d=%d: need B, n_new >= 0 and Hkv, d >= 1", B, Hkv, n_new, d);
  if (d % 16) return fail(FA_ERR_UNSUPPORTED, "d=%d: an FP8 row must be a multiple of 16 codes", d);
  if (!(k_scale > 0.f) || !isfinite(k_scale) || !(v_scale > 0.f) || !isfinite(v_scale))
    return fail(FA_ERR_INVALID, "k_scale and v_scale must be finite and > 0");
  int st0 = check_cache_layout(block_table, block_size, max_blocks_per_seq, kv_capacity, 0);
  if (st0 != FA_OK) return st0;
  if (B == 0 || n_new == 0) return ok();
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return fail(FA_ERR_INVALID, "null tensor pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(FA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) & 3u) return fail(FA_ERR_INVALID, "seq_lens must be 4-byte aligned");
  if ((long long)B * Hkv > 65535) return fail(FA_ERR_UNSUPPORTED, "B * Hkv must be <= 65535");
  if ((long long)n_new * (d / 16) > 0x7fffffffll) return fail(FA_ERR_UNSUPPORTED, "n_new too large");

  fa::AppendArgs a{};
  a.k_new = k_new; a.v_new = v_new; a.k = k_cache; a.v = v_cache;
  a.seq_lens = seq_lens; a.block_table = block_table;
  a.block_size = block_table ? block_size : 0;
  a.log2_block_size = block_table ? ilog2(block_size) : 0;
  a.max_blocks_per_seq = block_table ? max_blocks_per_seq : 0;
  a.kv_capacity = kv_capacity;
  a.B = B; a.Hkv = Hkv; a.n_new = n_new; a.row_chunks = d / 16;
  a.quantize = 1; a.k_scale = k_scale; a.v_scale = v_scale;
  hipError_t e = fa::launch_kv_append(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
