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
// A copy, bound by HBM bandwidth: one lane moves one 16-byte chunk of K and
// the matching chunk of V (into an FP8 cache: 16 bf16 values quantised to 16
// E4M3 codes; the per-tensor scale convention is the library's reading, the
// pages only say that the cache may hold one byte per number).  Consecutive lanes take consecutive chunks of a
// (head, token) row, so both the reads of the new rows and the writes into the
// cache are whole 16-byte-aligned runs of d elements.  A sequence whose length
// breaks the contract, or a block id outside the pool, is skipped: nothing is
// ever written outside the cache.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// 16 bf16 (two 16-byte vectors) -> 16 E4M3 codes (one 16-byte vector): each
// value is divided by `scale` in fp32 (IEEE division), saturated to +-448
// (E4M3's largest magnitude; a NaN stays NaN) and rounded to the nearest code,
// ties to even, by v_cvt_pk_fp8_f32.
__device__ __forceinline__ u32x4_t quantize16(const u32x4_t& x0, const u32x4_t& x1, float scale) {
  u32x4_t out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4_t& x = w < 2 ? x0 : x1;
    const uint32_t d0 = x[(w % 2) * 2], d1 = x[(w % 2) * 2 + 1];
    float f[4] = {bf16lo_to_f32(d0), bf16hi_to_f32(d0), bf16lo_to_f32(d1), bf16hi_to_f32(d1)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = f[i] / scale;
      f[i] = y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);
    out[w] = (uint32_t)r;
  }
  return out;
}

// grid: x over the (token, chunk) pairs of one (sequence, KV head), y = b * Hkv + g.
// A chunk is 16 bytes of the cache row: 16 codes (FP8) read from 32 bytes of
// bf16, or 16 bytes copied.
template <bool QUANT>
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
  u32x4_t kv, vv;
  if constexpr (QUANT) {
    const u32x4_t* kn = reinterpret_cast<const u32x4_t*>(a.k_new) + 2 * src;
    const u32x4_t* vn = reinterpret_cast<const u32x4_t*>(a.v_new) + 2 * src;
    kv = quantize16(__builtin_nontemporal_load(kn), __builtin_nontemporal_load(kn + 1), a.k_scale);
    vv = quantize16(__builtin_nontemporal_load(vn), __builtin_nontemporal_load(vn + 1), a.v_scale);
  } else {
    kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.k_new) + src);
    vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.v_new) + src);
  }

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
  if (a.quantize)
    hipLaunchKernelGGL(kv_append_kernel<true>, dim3((unsigned)bx, (unsigned)by), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<false>, dim3((unsigned)bx, (unsigned)by), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
