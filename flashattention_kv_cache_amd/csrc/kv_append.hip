// KV-cache append: the keys and values of n_new new tokens per sequence are
// written into the cache, at positions L_b - n_new .. L_b - 1 (L_b = the
// sequence's length after the append).
//
// Paged layout: token t of a sequence lives in slot t % block_size of physical
// block block_table[t / block_size] of a pool shaped (num_blocks, block_size,
// Hkv, d) ("Module 09: Efficient Attention", section "Code: A Paged KV Cache
// from Scratch").  The blocks themselves are claimed by the caller's allocator
// before the call: the table already lists them.
//
// A pure copy, bound by HBM bandwidth: one lane moves one 16-byte chunk of K
// and the matching chunk of V.  Consecutive lanes take consecutive chunks of a
// (head, token) row, so both the reads of the new rows and the writes into the
// cache are whole 16-byte-aligned runs of d elements.  A sequence whose length
// breaks the contract, or a block id outside the pool, is skipped: nothing is
// ever written outside the cache.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// grid: x over the (token, chunk) pairs of one (sequence, KV head), y = b * Hkv + g
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a) {
  const unsigned idx = blockIdx.x * kThreads + threadIdx.x;
  const unsigned per_head = (unsigned)a.n_new * (unsigned)a.row_chunks;
  if (idx >= per_head) return;
  const int c = (int)(idx % (unsigned)a.row_chunks);
  const int i = (int)(idx / (unsigned)a.row_chunks);
  const int b = (int)(blockIdx.y / (unsigned)a.Hkv);
  const int g = (int)(blockIdx.y % (unsigned)a.Hkv);

  // the new rows first: their addresses need no lookup, so they fly while the
  // length and the block id arrive
  const size_t src = (size_t)blockIdx.y * per_head + idx;
  const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new) + src);
  const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new) + src);

  const int L = a.seq_lens[b];
  const long long cap = a.block_table ? (long long)a.max_blocks_per_seq * a.block_size : (long long)a.kv_capacity;
  if (L < a.n_new || L > cap) return;
  const int t = L - a.n_new + i;

  size_t dst_row;  // (token, head) row of the cache, in units of d elements
  if (a.block_table) {
    const int blk = a.block_table[(size_t)b * a.max_blocks_per_seq + (t >> a.log2_block_size)];
    if (blk < 0 || blk >= a.kv_capacity) return;
    dst_row = ((size_t)blk * a.block_size + (t & (a.block_size - 1))) * a.Hkv + g;
  } else {
    dst_row = ((size_t)b * a.Hkv + g) * a.kv_capacity + t;
  }
  const size_t dst = dst_row * a.row_chunks + c;
  reinterpret_cast<u32x4_t*>(a.k)[dst] = kv;
  reinterpret_cast<u32x4_t*>(a.v)[dst] = vv;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const long long per_head = (long long)a.n_new * a.row_chunks;
  const long long bx = (per_head + kThreads - 1) / kThreads;
  const long long by = (long long)a.B * a.Hkv;
  if (per_head > 0x7fffffffll || bx > 0x7fffffff || by > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)bx, (unsigned)by), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
