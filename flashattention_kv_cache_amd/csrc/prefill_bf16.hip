// bf16 prefill on the gfx950 matrix cores: exact attention, streaming softmax,
// fp32 accumulation.
//
// The algorithm is the tiled one of "KV Cache, Flash Attention and Inference
// Optimization", section "the tiling trick": a workgroup loads its query tile
// once, walks the key/value tiles, forms the tile's scores on chip, folds them
// into a running softmax and accumulates the output tile, which is written to
// HBM once.  The running-softmax update is the recurrence of the "Li Hongyi,
// Machine Learning 2026" notes (lecture "FlashAttention": running max d_k,
// running sum s_k, earlier partials rescaled by e^{d_{k-1} - d_k}), kept in the
// unnormalised-accumulator form (one division at the end).
//
// gfx950 mapping (not from the pages):
//   * workgroup = 4 waves = 128 query rows; each wave owns 32 rows.  Key and
//     value tiles of 64 rows go from HBM straight into LDS with
//     global_load_lds_dwordx4 (no staging registers, no vector ALU work):
//     K and V each double buffered, staggered by one tile.
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries kept in
//     registers for the whole kernel.  In the accumulator layout a lane then
//     holds 16 keys of ONE query column (the other 16 sit in lane ^ 32), so a
//     row max is 15 in-lane maxima plus one v_permlane32_swap, and the row sum
//     stays a per-lane partial until the epilogue.
//   * the exponentiated scores, packed to bf16, are already the B operand of
//     O^T += V^T P^T (k = keys): register r of the S^T accumulator holds key
//     8*(r/4) + 4*(lane/32) + r%4, so the k index of the PV product is a fixed
//     permutation of the keys.  The V^T operand is read from the row-major V
//     tile with two ds_read_b64_tr_b16 (each gives a lane 4 keys of its
//     dimension); the rows they address follow the same permutation.
//   * LDS tiles are XOR-swizzled in 16-byte chunks (the swizzle is applied to
//     the source addresses of the direct loads): K by row % 8, so 16-byte
//     operand reads of 8 consecutive keys hit distinct banks; V by
//     2 * (row % 4), so each transposed read of 4 keys x 16 dims does.
//   * software pipeline inside each wave: iteration t runs the QK^T MFMAs of
//     tile t+1 interleaved with the softmax arithmetic of tile t (they are
//     independent), then the PV MFMAs of tile t; the direct loads of K(t+2)
//     and V(t+1) fly during the whole iteration.  One barrier per tile.
//   * causal: only key tiles left of and on the diagonal are visited, the mask
//     is evaluated only on tiles that cross the diagonal or the key tail, and
//     the grid is ordered longest query tiles first; workgroups that share a
//     KV head are placed on the same XCD (dispatch is round-robin over the 8
//     XCDs) so that head's K/V stays in that XCD's L2.
//   * the row sum is accumulated in fp32 from the unrounded weights (a sum of
//     the bf16-rounded weights would move the log-sum-exp by ~1e-3 on short
//     rows).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr float kSlack = 8.f;  // log2 units a running max may lag before rescaling

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

template <int D>
struct Smem {
  uint16_t k[2][kBN * D];  // row-major K tiles, chunks swizzled by row % 8
  uint16_t v[2][kBN * D];  // row-major V tiles, chunks swizzled by 2 * (row % 4)
};

__device__ __forceinline__ int k_swz(int row) { return row & 7; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 1; }

// Direct global -> LDS copy of tile rows [key0, key0 + 64) of one head.  A
// wave instruction writes 1 KiB of consecutive LDS (lane L at 16 L); lane L
// fetches the global chunk that the swizzle places there.  Rows at or past Nk
// are read from row Nk - 1 instead: harmless (keys >= Nk get weight 0 and the
// clamped V rows are finite) and never out of bounds.  Tiles past the last
// one are loaded the same way and never used.
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(const uint16_t* src, uint16_t* dst_tile, int key0, int Nk, int wave, int lane) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per wave instruction
  constexpr int IPW = kBN / RPI / 4;    // instructions per wave
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * RPI + lane / CPR;
    const int p = lane % CPR;
    const int c = p ^ (IS_V ? v_swz(row) : k_swz(row));
    const int key = min(key0 + row, Nk - 1);
    lds_u16* dst = (lds_u16*)(dst_tile + (wave * IPW + i) * RPI * D);
    __builtin_amdgcn_global_load_lds(src + (size_t)key * D + c * 8, dst, 16, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a, int nqb) {
  __shared__ Smem<D> sm;
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int VPS = 16 / KS; // softmax values of one 32-key block per QK^T k-step

  // ---- work item: (b, h, query tile), longest first, KV-head-major per XCD
  const int id = blockIdx.x;
  const int n_rep = a.Hq / a.Hkv;
  const int GP = a.B * a.Hkv;
  int b, h, qb;
  if ((GP & 7) == 0) {
    const int xcd = id & 7, j = id >> 3;
    const int per = (GP >> 3) * n_rep;  // work items per query-tile rank on one XCD
    const int rank = j / per, rest = j % per;
    const int gp = xcd + 8 * (rest / n_rep);
    b = gp / a.Hkv;
    h = (gp % a.Hkv) * n_rep + rest % n_rep;
    qb = nqb - 1 - rank;
  } else {
    const int rank = id / (a.B * a.Hq), bh = id % (a.B * a.Hq);
    b = bh / a.Hq;
    h = bh % a.Hq;
    qb = nqb - 1 - rank;
  }
  const int g = h / n_rep;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;   // which half of the wave
  const int col = lane & 31;  // query column within the wave's 32 rows
  const int q0 = qb * kBM;
  const int off = a.Nk - a.Nq;
  const int last_row = min(a.Nq, q0 + kBM) - 1;
  const int kend = a.causal ? min(a.Nk, last_row + off + 1) : a.Nk;
  const int n_tiles = (kend + kBN - 1) / kBN;
  // tiles below this index need no mask for any row of the workgroup
  const int n_clean = a.causal ? min((q0 + off + 1) / kBN, a.Nk / kBN) : a.Nk / kBN;

  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + (size_t)(b * a.Hkv + g) * a.Nk * D;

  // ---- Q^T operand fragments, kept in registers
  const int qrow = q0 + wave * 32 + col;
  bf16x8_t qf[KS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq + min(qrow, a.Nq - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16 + hl * 8);
  }

  f32x16_t oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m = -INFINITY, l0 = 0.f, l1 = 0.f;
  const float c = a.scale * kLog2e;

  // LDS element offset of this lane's K operand (row kb*32 + col, logical
  // 16-byte chunk ks*2 + hl), and of its V^T transposed reads.
  auto k_off = [&](int kb, int ks) {
    const int row = kb * 32 + col;
    return row * D + (((ks * 2 + hl) ^ k_swz(row)) * 8);
  };
  // V^T operand for k-step kk (keys 16kk .. 16kk+15) and dims db*32 .. +31:
  // lane L of 16-lane group gi reads row key(j) = 16kk + 8*half + 4*(gi/2) + j
  // with j = (L%16)/4, at dims db*32 + 16*(gi%2) + 4*(L%4) .. +3; the
  // transpose hands lane L the 4 keys of dim db*32 + L%32.
  const int gi = lane >> 4, li = lane & 15;
  auto v_off = [&](int kk, int half, int db) {
    const int row = kk * 16 + half * 8 + (gi >> 1) * 4 + (li >> 2);
    const int d = db * 32 + (gi & 1) * 16 + (li & 3) * 4;
    return row * D + ((((d >> 3) ^ v_swz(row)) << 3) | (d & 7));
  };

  // S^T of one tile for this wave's 32 queries: two 32-key blocks
  auto qk = [&](f32x16_t (&sacc)[2], int buf) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&sm.k[buf][k_off(kb, ks)]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16_t{} : sacc[kb], 0, 0, 0);
      }
  };
  // Keys past Nk and, when causal, keys right of the (bottom-right aligned)
  // diagonal get weight 0.  Register r of block kb holds key
  // t*64 + kb*32 + 8*(r/4) + 4*hl + r%4, so one compare against a per-lane
  // limit decides each element.
  auto mask = [&](f32x16_t (&sacc)[2], int t) {
    const int lim = (a.causal ? min(qrow + off, a.Nk - 1) : a.Nk - 1) - (t * kBN + hl * 4);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + (r / 4) * 8 + (r % 4) > lim) sacc[kb][r] = -INFINITY;
  };

  // One pipeline stage: softmax + PV of tile t (scores in sc), QK^T of tile
  // t+1 into sn, direct loads of K(t+2) and V(t+1) in flight.
  auto stage = [&](f32x16_t (&sc)[2], f32x16_t (&sn)[2], int t) {
    const int cb = t & 1;  // buffer holding V(t); K(t+1) sits in cb ^ 1
    dma_tile<D, false>(kg, sm.k[cb], (t + 2) * kBN, a.Nk, wave, lane);
    dma_tile<D, true>(vg, sm.v[cb ^ 1], (t + 1) * kBN, a.Nk, wave, lane);

    // ---- part A: mask, running max, rare rescale
    if (t >= n_clean) mask(sc, t);
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    mx = halves_max(mx) * c;
    // Rescale only when some row's max grows by more than kSlack (log2
    // units): (m, l, O) stays exact for any reference m within kSlack of the
    // true max, and P is then at most 2^kSlack (fine in bf16).
    const float mn = fmaxf(m, mx);
    if (__any(mn > m + kSlack)) {
      const float alpha = fast_exp2(m - ((mn == -INFINITY) ? 0.f : mn));
      l0 *= alpha;
      l1 *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m = mn;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;

    // ---- part B: S(t+1) on the matrix cores, P(t) on the vector ALUs
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&sm.k[cb ^ 1][k_off(kb, ks)]);
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16_t{} : sn[kb], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < VPS; ++j) {
          const int r = ks * VPS + j;
          p[r] = fast_exp2(fmaf(sc[kb][r], c, -mu));
          if (j & 1) l1 += p[r]; else l0 += p[r];
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(p[half * 8 + 2 * i], p[half * 8 + 2 * i + 1]);
        pf[kb * 2 + half] = __builtin_bit_cast(bf16x8_t, w);
      }
    }

    // ---- part C: O^T += V(t)^T P(t)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[cb] + v_off(kk, 0, db)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[cb] + v_off(kk, 1, db)));
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kk], oacc[db], 0, 0, 0);
      }
    wait_all_vmem();  // this wave's direct loads have landed
    __syncthreads();  // ... and every other wave's
  };

  f32x16_t s_a[2], s_b[2];
  if (n_tiles > 0) {
    // prologue: K(0), V(0) -> buffer 0, K(1) -> K buffer 1
    dma_tile<D, false>(kg, sm.k[0], 0, a.Nk, wave, lane);
    dma_tile<D, true>(vg, sm.v[0], 0, a.Nk, wave, lane);
    dma_tile<D, false>(kg, sm.k[1], kBN, a.Nk, wave, lane);
    wait_all_vmem();
    __syncthreads();
    qk(s_a, 0);
    __syncthreads();  // K buffer 0 is refilled by the first stage
  }
  for (int t = 0; t < n_tiles; t += 2) {
    stage(s_a, s_b, t);
    if (t + 1 >= n_tiles) break;
    stage(s_b, s_a, t + 1);
  }

  // ---- epilogue: one division, bf16 output, natural-log LSE
  const float lt = halves_sum(l0 + l1);
  if (qrow >= a.Nq) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* op = reinterpret_cast<uint16_t*>(a.o) + ((size_t)(b * a.Hq + h) * a.Nq + qrow) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + q4 * 8 + hl * 4;
      u32x2_t w;
      w[0] = pack_bf16x2(oacc[db][q4 * 4 + 0] * inv, oacc[db][q4 * 4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][q4 * 4 + 2] * inv, oacc[db][q4 * 4 + 3] * inv);
      *reinterpret_cast<u32x2_t*>(op + d) = w;
    }
  if (a.lse && hl == 0)
    a.lse[(size_t)(b * a.Hq + h) * a.Nq + qrow] = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + kBM - 1) / kBM;
  const long long grid = (long long)nqb * a.Hq * a.B;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (a.d == 64)
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, nqb);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, nqb);
  return hipGetLastError();
}

}  // namespace fa
