// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// ---------------------------------------------------------------------------
// Launch descriptors (host side fills, launchers consume).
// ---------------------------------------------------------------------------
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  int causal;
  int window;  // > 0: a causal query sees only its `window` most recent keys
  float scale;
  // Keys read from a KV cache (chunked prefill).  seq_lens == nullptr: plain
  // prefill, Nk keys per head stored (B, Hkv, Nk, d).  Otherwise sequence b has
  // seq_lens[b] cached keys, the Nq queries are its newest tokens, and K/V are
  // a contiguous cache (B, Hkv, kv_capacity, d) when block_table == nullptr,
  // else a pool (kv_capacity blocks, block_size, Hkv, d) read through
  // block_table (B, max_blocks_per_seq).
  const int32_t* seq_lens;
  const int32_t* block_table;
  int block_size, log2_block_size, max_blocks_per_seq;
  int kv_capacity, max_seq_len;
};

struct AppendArgs {
  const void* k_new;           // (B, Hkv, n_new, d)
  const void* v_new;
  void* k;                     // contiguous (B, Hkv, kv_capacity, d) or pool (kv_capacity, bs, Hkv, d)
  void* v;
  const int32_t* seq_lens;     // (B) lengths after the append
  const int32_t* block_table;  // nullptr: contiguous
  int block_size, log2_block_size, max_blocks_per_seq, kv_capacity;
  int B, Hkv, n_new, row_chunks;  // row_chunks: 16-byte chunks per (token, head) row of the cache
  int quantize;                   // 1: bf16 rows into an FP8 (E4M3) cache, code = RNE(x / scale)
  float k_scale, v_scale;
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* block_table;  // nullptr: contiguous layout
  int block_size, log2_block_size, max_blocks_per_seq;
  int kv_capacity, max_seq_len;
  int window;         // > 0: only the last `window` keys of each sequence
  void* o;
  float* lse;
  int B, Hq, Hkv, d;
  float scale;
  float k_scale, v_scale;  // FP8 caches: a code stands for value(code) * scale (1 otherwise)
  int split_tokens;   // tokens per split (multiple of 256)
  int max_splits;     // ceil(max_seq_len / split_tokens), >= 1
  float* ws_o;        // (B, Hq, max_splits, d) partial outputs, when max_splits > 1
  float* ws_lse;      // (B, Hq, max_splits) partial log-sum-exp
  int32_t* plan;      // 1 + B * max_splits: count, then b * max_splits + s, longest first (max_splits > 1)
};

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
struct MlaArgs {
  const void* q;               // (B, Hq, DC + DR) bf16: [absorbed content query ; position query]
  const void* kv;              // rows [latent ; position key]: contiguous (B, kv_capacity, DC + DR) or
                               // a pool (kv_capacity blocks, block_size, DC + DR), bf16
  const int32_t* seq_lens;
  const int32_t* block_table;  // nullptr: contiguous
  int block_size, log2_block_size, max_blocks_per_seq, kv_capacity, max_seq_len;
  void* o;                     // (B, Hq, DC) bf16
  float* lse;                  // (B, Hq) or nullptr
  int B, Hq;
  float scale;
  int split_tokens, max_splits;
  uint16_t* ws_o;              // (B, Hq, max_splits, DC) bf16 partial outputs, when max_splits > 1
  float* ws_lse;               // (B, Hq, max_splits)
  int32_t* plan;               // 1 + B * max_splits: count, then b * max_splits + s, longest first
};
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t s);

enum class KvType { F32, BF16, FP8 };  // cache element type (queries/outputs: fp32, bf16, bf16)
hipError_t launch_decode(const DecodeArgs& a, KvType t, hipStream_t s);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values packed into one dword
// (lo = a, hi = b); gfx950 has a single instruction for it.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r = {(__bf16)a, (__bf16)b};  // lowers to v_cvt_pk_bf16_f32
  return __builtin_bit_cast(uint32_t, r);
}

// DPP lane exchanges inside a row of 16 lanes.
enum : int {
  kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,  // lane i <-> 7-i within each 8 lanes
  kDppMirror = 0x140,      // lane i <-> 15-i within each 16 lanes
  kDppRor8 = 0x128,        // rotate right by 8 within each 16 lanes
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another.  Applied to two copies of x, lane l ends up holding the
// pair {x[l % 32], x[l % 32 + 32]} across the two results, so the max and the
// sum of the two are the combine of lane l with lane l ^ 32 (whichever result
// holds which half).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maximum that propagates NaN (v_maximum3_f32 on gfx950).  Unlike fmaxf it
// needs no canonicalising v_max of each operand in IEEE mode; a NaN score
// makes its row NaN either way.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float halves_max_nan(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reinterpret a dword as two bf16.  Goes through a scalar copy: this clang
// miscompiles __builtin_bit_cast applied directly to an ext_vector element
// subscript (it reads element 0 whatever the index).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  bf16x2_t r;
  __builtin_memcpy(&r, &w, sizeof r);
  return r;
}

// Work lists of the split-K decode kernels: a one-workgroup counting sort of
// the (sequence, split) items by length, longest first.  The counts sit in
// kPlanBuckets LDS counters, bucket 0 the longest; this turns them into
// exclusive start offsets (4 buckets a thread, a scan across lanes, then
// across waves) and returns the number of items.  All kPlanThreads threads
// call it; it ends with a barrier.
constexpr int kPlanThreads = 256, kPlanBuckets = 1024;
__device__ __forceinline__ int plan_exclusive_scan(int* cnt) {
  static_assert(kPlanBuckets == 4 * kPlanThreads && kPlanThreads % 64 == 0, "plan scan shape");
  __shared__ int wave_total[kPlanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c0 = cnt[4 * t], c1 = cnt[4 * t + 1], c2 = cnt[4 * t + 2], c3 = cnt[4 * t + 3];
  const int own = c0 + c1 + c2 + c3;
  int incl = own;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kPlanThreads / 64; ++w) {
    if (w < wave) base += wave_total[w];
    total += wave_total[w];
  }
  const int run = base + incl - own;
  cnt[4 * t] = run;
  cnt[4 * t + 1] = run + c0;
  cnt[4 * t + 2] = run + c0 + c1;
  cnt[4 * t + 3] = run + c0 + c1 + c2;
  __syncthreads();
  return total;
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum, i.e. not waited).
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// LDS tiles of the MFMA kernels.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// Forces a value to be computed at this point of the program (an empty asm
// that reads it; no instruction is emitted).  Used so that the softmax of a
// tile is not sunk past the barrier into the next stage, where it could no
// longer overlap this stage's MFMAs.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(const u32x4_t& x) { asm volatile("" ::"v"(x)); }

// Direct global -> LDS copies (global_load_lds_dwordx4).  A wave instruction
// writes 1 KiB of consecutive LDS starting at M0 (lane L at 16 L); lane L
// fetches the global chunk that the kernel's swizzle places there.
//
// They are issued from inline assembly on purpose: the compiler cannot tell
// which LDS bytes such a load writes, and would otherwise drain every one of
// them (s_waitcnt vmcnt(0)) before the next transposed LDS read, i.e. in the
// middle of the tile that overlaps them.  The instruction writes no VGPR, so
// no register can be reused under it; the kernel itself waits for all of
// them (wait_all_vmem) before the barrier that publishes the tile, and
// vector-memory loads retire in order, so the compiler's own waits for other
// loads stay correct (only stricter).  M0 is written in the same block and
// declared clobbered; s_nop 0 covers the M0-write -> LDS-DMA hazard.
//
// NT = true sets the non-temporal bit: for data read once per launch (a KV
// cache streamed by decode), which then does not displace reusable lines in L2.
template <bool NT = false>
__device__ __forceinline__ void lds_dma_saddr(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
template <bool NT = false>
__device__ __forceinline__ void lds_dma_vaddr(const void* vaddr, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(vaddr), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(vaddr), "s"(lds_addr) : "memory", "m0");
}


}  // namespace fa
