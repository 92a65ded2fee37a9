// Multi-head latent attention (MLA) decode on the gfx950 matrix cores.
//
// What is computed ("Module 09: Efficient Attention", sections "The Math:
// Compress, Reconstruct, Decouple" and "Why RoPE Has To Be Decoupled"): the
// cache holds, per token, one row [c ; k^R] — the latent (DC = 512 numbers)
// and the decoupled position key (DR = 64) — shared by every head.  With the
// content query absorbed into latent space (q^lat_h = W^UK_h^T q^C_h, done by
// the caller), head h scores token j as [q^lat_h ; q^R_h] . [c_j ; k^R_j]
// times `scale` (the page: 1 / sqrt(d_head + d_r)), and its output is the
// softmax-weighted sum of the latents c_j, in latent space (the caller applies
// W^UV_h afterwards).  So every head attends one shared key of width 576 and
// one shared value of width 512 — the first 512 numbers of the same row.
//
// With 128 heads per token this is a dense contraction (4 flop per head per
// cached number, ~128 flop per cached byte), so it runs on MFMA
// (v_mfma_f32_16x16x32_bf16):
//   * a workgroup (8 waves, two per SIMD) takes 128 heads of one sequence and
//     one split of its tokens; wave w owns heads 16w .. 16w + 15.  Q^T
//     (576 x 16) of a wave stays in registers as the B operand of S^T = K Q^T
//     (2 key blocks x 18 k-steps per 32-key tile); O^T (512 x 16, fp32, 128
//     registers) accumulates O^T += V^T P^T (32 dim blocks, one k-step of all
//     32 keys).  Sixteen heads per wave keep the wave within 256 registers;
//     32 would need 256 accumulators alone;
//   * 32-key tiles of cache rows go HBM -> LDS with global_load_lds_dwordx4,
//     one tile serves both products (V is a prefix of K); the loads carry the
//     non-temporal bit, since each row is read once per call;
//   * rows are 72 sixteen-byte units; unit u of row r sits at u ^ (r % 8)
//     (low three bits only).  Measured with the LDS bank-conflict counter on
//     MI355X, this keeps both the K operand reads (16 rows at one unit) and
//     the transposed V reads (8 rows x 2 units) free of conflicts at this
//     1152-byte row stride, where other XOR patterns conflict 2- to 4-way;
//   * four tile buffers: tiles t + 1 .. t + 3 load while tile t is computed
//     (three tiles in flight per CU), one barrier per tile; a split's block
//     ids are staged in LDS first, so no vector-memory wait of the loop can
//     stall on tile loads in flight;
//   * the S^T accumulator gives a lane keys 4 g + i and 16 + 4 g + i (g = lane
//     / 16) of its head: packed in that order they are the B operand of PV as
//     they stand, and the transposed V reads fetch the same key rows;
//   * the streaming softmax (running max with a lazy rescale, fp32 row sum of
//     the unrounded weights, bf16 weights into PV) is the prefill kernel's;
//   * splits of a sequence write (output, log-sum-exp) partials that a merge
//     kernel combines with weights exp(lse_s - max lse); the normalised
//     partial outputs are stored in bf16 (the output's own precision), their
//     log-sum-exps in fp32.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDC = 512, kDR = 64, kDK = kDC + kDR;  // latent, position key, key width
constexpr int kUnits = kDK / 8;                       // 16-byte units per cache row (72)
constexpr int kBN = 32;                               // keys per tile
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kHeadsWave = 16, kHeadsWG = kHeadsWave * kWaves;  // 16 per wave, 128 per workgroup
constexpr int kKS = kDK / 32;                         // k-steps of S^T = K Q^T (18)
constexpr int kDB = kDC / 16;                         // 16-row blocks of O^T (32)
constexpr int kInstr = kBN * kUnits / 64;             // direct loads per tile (36)
constexpr int kBufs = 4;                              // tile buffers
constexpr int kMaxEntries = 1040;                     // staged block ids (16384 tokens / 16 + slack)
constexpr float kSlack = 8.f;                         // log2 units a running max may lag

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Physical unit of logical unit u in row r: only the low three bits move.
__device__ __forceinline__ int swz(int r) { return r & 7; }

struct alignas(16) Smem {
  uint16_t kv[kBufs][kBN * kDK];  // 4 x 36 KiB
  int32_t ent[kMaxEntries];       // block ids of the split (paged, block_size >= 16)
};

// MFMA steps issued from assembly, so that their order against the operand
// reads is the one written here (the compiler would otherwise hoist all of a
// tile's LDS reads ahead of the chain, out of registers).  Each accumulates in
// place (destination exactly overlapping SrcC, which the hardware forwards).
// What the compiler cannot see through the assembly is padded explicitly:
// vector instructions read an MFMA result (or overwrite its SrcC) only after
// mfma_done(), and an MFMA reads vector-written operands after valu_done().
__device__ __forceinline__ void mfma_first(f32x4& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_done(f32x4 (&acc)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]));
}
__device__ __forceinline__ void valu_done(bf16x8_t& p) { asm volatile("s_nop 3" : "+v"(p)); }
// Orders an LDS operand read after the MFMA issued before it: an empty
// statement that claims to change the read's base address in place (no copy,
// no arithmetic), so the read cannot move above it, and the read's own offset
// stays an immediate.
__device__ __forceinline__ void after_prev(uint32_t& addr) { asm volatile("" : "+v"(addr)); }
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
__device__ __forceinline__ const lds_bf16x8* lds_ptr(uint32_t addr) {
  return reinterpret_cast<const lds_bf16x8*>((uintptr_t)addr);
}

// Waves issue the 36 direct loads of a tile round-robin: wave w takes loads
// w, w + 8, ...; waves 0-3 issue 5, waves 4-7 issue 4.  s_waitcnt vmcnt(n),
// other counters not waited: all but this wave's last n vector-memory
// operations (the loads of its `younger` most recent tiles) are done.
__device__ __forceinline__ void wait_all_but_last_tiles(int wave, int younger) {
  if (wave < kInstr % kWaves) {
    if (younger >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (kInstr / kWaves + 1)));
    else if (younger == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (kInstr / kWaves + 1));
    else wait_all_vmem();
  } else {
    if (younger >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * (kInstr / kWaves)));
    else if (younger == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (kInstr / kWaves));
    else wait_all_vmem();
  }
}

// With several splits, a sequence of L tokens is cut into ns = ceil(L /
// split_tokens) equal parts of sl = ceil(L / ns) tokens, rounded up to a tile
// (sl <= split_tokens, and every part is non-empty), and the work items
// (sequence, part) are dispatched longest first from the list the plan
// kernel writes: one workgroup per CU takes them as CUs free up.
__device__ __forceinline__ int split_len(int L, int ns) {
  return ns <= 1 ? L : ((L + ns - 1) / ns + kBN - 1) / kBN * kBN;
}
__device__ __forceinline__ int split_count(const MlaArgs& a, int L) {
  const bool bad = L < 0 || L > a.max_seq_len;
  return bad ? 1 : max(1, (L + a.split_tokens - 1) / a.split_tokens);
}

// One workgroup: the list of work items sorted by tile count, longest first
// (a counting sort; the order among equal counts is free, and no result
// depends on it).  plan[0] = number of items.
__global__ __launch_bounds__(kPlanThreads) void mla_plan_kernel(MlaArgs a) {
  __shared__ int cnt[kPlanBuckets];
  for (int i = threadIdx.x; i < kPlanBuckets; i += kPlanThreads) cnt[i] = 0;
  __syncthreads();
  auto bucket = [&](int L, int ns, int s) {
    if (L < 0 || L > a.max_seq_len) return 0;
    const int sl = split_len(L, ns), t0 = s * sl, t1 = min(L, t0 + sl);
    return min(kPlanBuckets - 1, (t1 - t0 + kBN - 1) / kBN);
  };
  for (int b = threadIdx.x; b < a.B; b += kPlanThreads) {
    const int L = a.seq_lens[b], ns = split_count(a, L);
    for (int s = 0; s < ns; ++s) atomicAdd(&cnt[kPlanBuckets - 1 - bucket(L, ns, s)], 1);
  }
  __syncthreads();
  const int total = plan_exclusive_scan(cnt);
  if (threadIdx.x == 0) a.plan[0] = total;
  for (int b = threadIdx.x; b < a.B; b += kPlanThreads) {
    const int L = a.seq_lens[b], ns = split_count(a, L);
    for (int s = 0; s < ns; ++s) {
      const int pos = atomicAdd(&cnt[kPlanBuckets - 1 - bucket(L, ns, s)], 1);
      a.plan[1 + pos] = b * a.max_splits + s;
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void mla_split_kernel(MlaArgs a) {
  __shared__ Smem sm;
  const int hg = blockIdx.z;
  int s = 0, b = blockIdx.y;
  if (a.plan) {  // several splits: the work item from the longest-first list
    if ((int)blockIdx.x >= a.plan[0]) return;
    const int item = a.plan[1 + blockIdx.x];
    b = item / a.max_splits;
    s = item % a.max_splits;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, col = lane & 15;

  const int L = a.seq_lens[b];
  bool bad = L < 0 || L > a.max_seq_len;
  const int ns = split_count(a, L);
  if (s >= ns) return;
  const int sl = split_len(L, ns);
  const int t_begin = bad ? 0 : s * sl;
  const int t_end = bad ? 0 : min(L, t_begin + sl);
  const int n_tiles = (t_end - t_begin + kBN - 1) / kBN;

  const int h = hg * kHeadsWG + wave * kHeadsWave + col;  // this lane's head
  const bool wave_live = hg * kHeadsWG + wave * kHeadsWave < a.Hq;

  // ---- Q^T operand fragments: head h, dims 32 ks + 8 g .. + 7
  bf16x8_t qf[kKS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + min(h, a.Hq - 1)) * kDK + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 32);
  }
  // Drain here: otherwise the compiler's waits for these loads land inside
  // the tile loop, where (blind to the direct loads in flight) they would
  // drain the next tiles' loads every iteration.
  wait_all_vmem();
  f32x4 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l0 = 0.f, l1 = 0.f;
  const float c = a.scale * kLog2e;
  // the wait states vector instructions need before touching O^T after the
  // MFMAs that accumulate it
  auto oacc_done = [&]() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < kDB; ++i) asm volatile("" : "+v"(oacc[i]));
  };

  // ---- tile copy.  Load i of a tile fills units 64 i .. 64 i + 63 of the
  // tile's 32 x 72 units; lane L takes unit u = 64 i + L: row u / 72, physical
  // unit u % 72, whose logical unit it fetches.  A paged tile lies in one block
  // when block_size >= 32, and in two (rows 0-15: loads 0-17, rows 16-31: loads
  // 18-35) when block_size is 16; smaller blocks and the split's last tile
  // take the per-lane path.
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv);
  const int32_t* trow = a.block_table ? a.block_table + (size_t)b * a.max_blocks_per_seq : nullptr;
  const int bs = a.block_size, lbs = a.log2_block_size;
  // paged with blocks of >= 16 tokens: the split's block ids go to LDS once
  // (validated there); the tile loads then read them from LDS
  const int e_lo = trow && n_tiles > 0 ? t_begin >> lbs : 0;
  const int n_ent = trow && n_tiles > 0 ? ((t_end - 1) >> lbs) - e_lo + 1 : 0;
  const bool staged = trow && bs >= 16 && n_ent <= kMaxEntries;
  const bool blocky = trow == nullptr || staged;
  if (staged) {
    for (int i = threadIdx.x; i < n_ent; i += kThreads) {
      int e = trow[e_lo + i];
      if (e < 0 || e >= a.kv_capacity) { bad = true; e = 0; }
      sm.ent[i] = e;
    }
  }
  auto lds_of = [&](int buf) { return (uint32_t)(uintptr_t)(const lds_u16*)sm.kv[buf]; };
  auto entry = [&](int tok) { return sm.ent[(min(tok, t_end - 1) >> lbs) - e_lo]; };
  // Byte offset, within its block's rows, of the unit this lane fetches in
  // each of the wave's loads of a whole tile (the tile's rows 16-31 start a
  // second block when block_size is 16).
  constexpr int kLoadsWave = (kInstr + kWaves - 1) / kWaves;
  uint32_t dma_off[kLoadsWave];
#pragma unroll
  for (int k = 0; k < kLoadsWave; ++k) {
    const int i = min(wave + kWaves * k, kInstr - 1);
    const int u = 64 * i + lane, r = u / kUnits, p = u - r * kUnits;
    const int half = trow && bs == 16 ? i / (kInstr / 2) : 0;
    dma_off[k] = (uint32_t)(((r - 16 * half) * kDK + (p ^ swz(r)) * 8) * 2);
  }
  auto copy_tile = [&](int t, int buf) {
    const int tok0 = t_begin + t * kBN;
    const uint32_t lds0 = lds_of(buf);
    // The per-lane unit arithmetic of the partial-tile path below is cheap;
    // recomputing it per tile (the empty asm hides that it is loop-invariant)
    // keeps registers free.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (blocky && tok0 + kBN <= t_end) {
      int e0 = 0, e1 = 0;
      if (trow) {
        e0 = __builtin_amdgcn_readfirstlane(entry(tok0));
        e1 = __builtin_amdgcn_readfirstlane(entry(tok0 + 16));
      }
#pragma unroll
      for (int k = 0; k < (kInstr + kWaves - 1) / kWaves; ++k) {
        const int i = wave + kWaves * k;
        if (i >= kInstr) break;
        const uint16_t* base;
        if (trow) {
          const int half = bs == 16 ? i / (kInstr / 2) : 0;  // which block of the tile
          base = kv + ((size_t)(half ? e1 : e0) * bs + ((tok0 + 16 * half) & (bs - 1))) * kDK;
        } else {
          base = kv + ((size_t)b * a.kv_capacity + tok0) * kDK;
        }
        lds_dma_saddr<true>(dma_off[k], base, lds0 + i * 1024);
      }
    } else {
      // each lane finds its own token; rows past the split read its last
      // token (weight 0, finite)
#pragma unroll
      for (int k = 0; k < (kInstr + kWaves - 1) / kWaves; ++k) {
        const int i = wave + kWaves * k;
        if (i >= kInstr) break;
        const int u = 64 * i + ln, r = u / kUnits, p = u - r * kUnits;
        const int lu = p ^ swz(r);
        const int tok = min(tok0 + r, t_end - 1);
        size_t row;
        if (trow) {
          int blk = trow[tok >> lbs];
          if (blk < 0 || blk >= a.kv_capacity) { bad = true; blk = 0; }
          row = (size_t)blk * bs + (tok & (bs - 1));
        } else {
          row = (size_t)b * a.kv_capacity + tok;
        }
        lds_dma_vaddr<true>(kv + row * kDK + lu * 8, lds0 + i * 1024);
      }
    }
  };

  // LDS element offsets.  Only the low three bits of a unit index are
  // swizzled, so every offset is a lane-dependent base plus a constant.
  //   K operand of key block kb, k-step ks: row 16 kb + col, unit 4 ks + g,
  //     low bits 4 (ks % 2) + g -> kbase[kb][ks % 2] + 64 (ks / 2);
  //   V^T operand of dim block db: rows 4 g + j (keys 0-15 half) and
  //     16 + 4 g + j, dims 16 db + 4 a (j = lane % 16 / 4, a = lane % 4), unit
  //     2 db + a / 2, low bits 2 (db % 4) + a / 2 -> vbase[db % 4] + 64 (db / 4)
  //     (+ 16 rows for the second half).
  int kbase[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      kbase[kb][par] = (16 * kb + col) * kDK + (((4 * par + g) ^ swz(col)) << 3);
  // (recomputed where used, from a lane id the compiler cannot hoist)
  auto v_base = [&](int q) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int vrow = 4 * (ln >> 4) + ((ln & 15) >> 2), va = ln & 3;
    return vrow * kDK + (((2 * q + (va >> 1)) ^ swz(vrow)) << 3) + 4 * (va & 1);
  };

  // ---- prologue: block ids visible, tiles 0 - 2 in flight
  __syncthreads();
  if (n_tiles > 0) copy_tile(0, 0);
  if (n_tiles > 1) copy_tile(1, 1);
  if (n_tiles > 2) copy_tile(2, 2);

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & (kBufs - 1);
    // this wave's loads of tile t are done (those of tiles t + 1 and t + 2
    // may still fly) ...
    wait_all_but_last_tiles(wave, min(2, n_tiles - 1 - t));
    // ... and every wave's; every wave is also past tile t - 1, whose buffer
    // tile t + 3 now takes
    __syncthreads();
    if (t + 3 < n_tiles) copy_tile(t + 3, (t + 3) & (kBufs - 1));
    if (wave_live) {
      // LDS byte addresses of this lane's operands in the tile's buffer; each
      // read adds a constant as its immediate offset
      const uint32_t tile = lds_of(buf);
      // S^T = K Q^T: keys 16 kb + 4 g + i of head col in sacc[kb][i]
      // the two key blocks' chains alternate; each k-step's operands are
      // read while the previous step's MFMAs run
      uint32_t kaddr[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int par = 0; par < 2; ++par) kaddr[kb][par] = tile + 2 * kbase[kb][par];
      auto k_operand = [&](int kb, int ks) {
        after_prev(kaddr[kb][ks & 1]);
        return *lds_ptr(kaddr[kb][ks & 1] + 128 * (ks >> 1));
      };
      f32x4 sacc[2];
      bf16x8_t ka0 = k_operand(0, 0), ka1 = k_operand(1, 0);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        bf16x8_t na0 = ka0, na1 = ka1;
        if (ks + 1 < kKS) na0 = k_operand(0, ks + 1);
        if (ks == 0) mfma_first(sacc[0], ka0, qf[ks]);
        else mfma_acc(sacc[0], ka0, qf[ks]);
        if (ks + 1 < kKS) na1 = k_operand(1, ks + 1);
        if (ks == 0) mfma_first(sacc[1], ka1, qf[ks]);
        else mfma_acc(sacc[1], ka1, qf[ks]);
        ka0 = na0;
        ka1 = na1;
      }
      mfma_done(sacc);
      if (t == n_tiles - 1) {  // keys past the split get weight 0
        const int lim = t_end - 1 - (t_begin + t * kBN + 4 * g);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * kb + i > lim) sacc[kb][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                       fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = halves_max(mx) * c;  // the head's max over all 32 keys
      const float mn = fmaxf(m, mx);
      if (__any(mn > m + kSlack)) {
        const float alpha = fast_exp2(m - ((mn == -INFINITY) ? 0.f : mn));
        oacc_done();
#pragma unroll
        for (int i = 0; i < kDB; ++i) oacc[i] *= alpha;
        l0 *= alpha;
        l1 *= alpha;
        m = mn;
      }
      const float mu = (m == -INFINITY) ? 0.f : m;
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = fast_exp2(fmaf(sacc[kb][i], c, -mu));
          if (kb) l1 += p[kb][i]; else l0 += p[kb][i];
        }
      u32x4_t w;
      w[0] = pack_bf16x2(p[0][0], p[0][1]);
      w[1] = pack_bf16x2(p[0][2], p[0][3]);
      w[2] = pack_bf16x2(p[1][0], p[1][1]);
      w[3] = pack_bf16x2(p[1][2], p[1][3]);
      bf16x8_t pc = __builtin_bit_cast(bf16x8_t, w);
      valu_done(pc);
      // O^T += V^T P^T, one k-step of 32 keys per 16-dim block; each block's
      // operand is read while the two blocks before it run
      uint32_t vaddr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) vaddr[q] = tile + 2 * v_base(q);
      auto v_operand = [&](int db) {
        after_prev(vaddr[db & 3]);
        const uint32_t p = vaddr[db & 3] + 128 * (db >> 2);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)p);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(p + 2 * 16 * kDK));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t vq[3];  // operands of blocks db, db + 1 (read) and db + 2 (being read)
      vq[0] = v_operand(0);
      vq[1] = v_operand(1);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if (db + 2 < kDB) vq[(db + 2) % 3] = v_operand(db + 2);
        mfma_acc(oacc[db], vq[db % 3], pc);
      }
    }
  }

  // ---- epilogue
  oacc_done();
  const bool any_bad = __syncthreads_or(bad);
  float lt = l0 + l1;
  lt += __shfl_xor(lt, 16);
  lt = halves_sum(lt);
  if (!wave_live || h >= a.Hq) return;
  const float inv = any_bad ? __builtin_nanf("") : lt > 0.f ? 1.f / lt : 0.f;
  const float lse = any_bad ? __builtin_nanf("") : lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  if (ns == 1) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + ((size_t)b * a.Hq + h) * kDC + 4 * g;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      u32x2_t w2;
      w2[0] = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
      w2[1] = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
      *reinterpret_cast<u32x2_t*>(op + 16 * db) = w2;
    }
    if (a.lse && g == 0) a.lse[(size_t)b * a.Hq + h] = lse;
  } else {
    // the partial output in bf16 (normalised: within bf16 rounding of the
    // final output, which is bf16 too), its log-sum-exp in fp32: half the
    // partials' round trip through memory
    const size_t slot = ((size_t)b * a.Hq + h) * a.max_splits + s;
    uint16_t* op = a.ws_o + slot * kDC + 4 * g;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      u32x2_t w2;
      w2[0] = pack_bf16x2(oacc[db][0] * inv, oacc[db][1] * inv);
      w2[1] = pack_bf16x2(oacc[db][2] * inv, oacc[db][3] * inv);
      *reinterpret_cast<u32x2_t*>(op + 16 * db) = w2;
    }
    if (g == 0) a.ws_lse[slot] = lse;
  }
}

// One (sequence, head) per workgroup: the splits' outputs weighted by
// exp(lse_s - max_s lse_s).
__global__ __launch_bounds__(kDC / 4) void mla_merge_kernel(MlaArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int L = a.seq_lens[b];
  const bool bad = L < 0 || L > a.max_seq_len;
  const int ns = bad ? 1 : max(1, (L + a.split_tokens - 1) / a.split_tokens);
  if (ns == 1) return;  // written by the split kernel
  const size_t slot0 = (size_t)bh * a.max_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_lse[slot0 + s]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int e = threadIdx.x * 4;
  for (int s = 0; s < ns; ++s) {
    const float w = __expf(a.ws_lse[slot0 + s] - M);
    wsum += w;
    const u32x2_t p = *reinterpret_cast<const u32x2_t*>(a.ws_o + (slot0 + s) * kDC + e);
    acc[0] = fmaf(w, bf16lo_to_f32(p[0]), acc[0]);
    acc[1] = fmaf(w, bf16hi_to_f32(p[0]), acc[1]);
    acc[2] = fmaf(w, bf16lo_to_f32(p[1]), acc[2]);
    acc[3] = fmaf(w, bf16hi_to_f32(p[1]), acc[3]);
  }
  const float inv = 1.f / wsum;
  u32x2_t out;
  out[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  out[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.o) + (size_t)bh * kDC + e) = out;
  if (a.lse && threadIdx.x == 0) a.lse[bh] = M + __logf(wsum);
}

}  // namespace

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t st) {
  const int hgroups = (a.Hq + kHeadsWG - 1) / kHeadsWG;
  if (a.max_splits > 1) {
    hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
    hipLaunchKernelGGL(mla_split_kernel, dim3(a.B * a.max_splits, 1, hgroups), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(mla_split_kernel, dim3(1, a.B, hgroups), dim3(kThreads), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(a.B * a.Hq), dim3(kDC / 4), 0, st, a);
  return hipGetLastError();
}

}  // namespace fa
