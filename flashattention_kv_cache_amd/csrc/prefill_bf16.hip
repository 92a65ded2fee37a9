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
//   * workgroup = 4 waves = 128 query rows; each wave owns 32 rows.  Key/value
//     tiles of 64 rows are staged in LDS, double buffered, with the global
//     loads of tile t+1 in flight while tile t is computed.
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries kept in
//     registers for the whole kernel.  In the accumulator layout a lane then
//     holds 16 keys of ONE query column (the other 16 sit in lane ^ 32), so a
//     row max is 15 in-lane maxima plus one v_permlane32_swap, and the row sum
//     stays a per-lane partial until the epilogue.
//   * the exponentiated scores, packed to bf16, are already in the B-operand
//     layout of O^T += V^T P^T (k = keys): register r of the S^T accumulator
//     holds key 8*(r/4) + 4*(lane/32) + r%4, so the k index of the PV product
//     is a fixed permutation of the keys, and the V^T operand is read from LDS
//     in that same order.  V is transposed into LDS as groups of 4 keys per
//     dimension during staging, so each V^T operand is two 8-byte LDS reads.
//   * K rows in LDS are XOR-swizzled in 16-byte chunks so the 16-byte operand
//     reads of 16 consecutive keys hit distinct banks.
//   * causal: only key tiles left of and on the diagonal are visited, the mask
//     is evaluated only on tiles that cross the diagonal or the key tail, and
//     the grid is ordered longest query tiles first; workgroups that share a
//     KV head are placed on the same XCD (dispatch is round-robin over the 8
//     XCDs) so that head's K/V stays in that XCD's L2.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;

template <int D>
struct Smem {
  // K tile: 64 rows x D, row-major, 16-byte chunks XOR-swizzled per row.
  uint16_t k[2][kBN * D];
  // V tile transposed in groups of 4 keys: [key/4][d][key%4].
  uint16_t vt[2][kBN * D];
};

template <int D>
__device__ __forceinline__ int k_swz(int row, int chunk) {
  // D=128: 16 chunks per 256-byte row; D=64: 8 chunks per 128-byte row,
  // two rows per 256 bytes of banks.
  return chunk ^ ((row / (128 / D)) & (D / 8 - 1));
}

template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* kg, const uint16_t* vg, int key0, int Nk,
                                          u32x4_t (&kr)[D / 32], u32x4_t (&vr)[4]) {
  const int t = threadIdx.x;
  // K: each pass covers 2048 elements = 2048/D rows, 16 bytes per thread.
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const int row = p * (2048 / D) + t / (D / 8);
    const int col = (t % (D / 8)) * 8;
    const int key = key0 + row;
    kr[p] = key < Nk ? *reinterpret_cast<const u32x4_t*>(kg + (size_t)key * D + col) : u32x4_t{0, 0, 0, 0};
  }
  // V: thread handles 4 consecutive keys x 8 dims (2*D threads in use).
  if (t < 2 * D) {
    const int kgp = t / (D / 8), dc = t % (D / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = key0 + kgp * 4 + i;
      vr[i] = key < Nk ? *reinterpret_cast<const u32x4_t*>(vg + (size_t)key * D + dc * 8) : u32x4_t{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(Smem<D>& sm, int buf, const u32x4_t (&kr)[D / 32], const u32x4_t (&vr)[4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const int row = p * (2048 / D) + t / (D / 8);
    const int chunk = t % (D / 8);
    *reinterpret_cast<u32x4_t*>(&sm.k[buf][row * D + k_swz<D>(row, chunk) * 8]) = kr[p];
  }
  if (t < 2 * D) {
    const int kgp = t / (D / 8), dc = t % (D / 8);
    // vr[i] holds dims dc*8..dc*8+7 of key 4*kgp+i as 4 dwords of bf16 pairs.
    // Output: for each dim, the 4 keys as 2 dwords.
    u32x4_t out[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims 2w (lo halves) and 2w+1 (hi halves)
      const uint32_t lo01 = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
      const uint32_t lo23 = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
      const uint32_t hi01 = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
      const uint32_t hi23 = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
      out[w] = u32x4_t{lo01, lo23, hi01, hi23};
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&sm.vt[buf][(kgp * D + dc * 8) * 4]);
#pragma unroll
    for (int w = 0; w < 4; ++w) dst[w] = out[w];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillArgs a, int nqb) {
  __shared__ Smem<D> sm;
  constexpr int KS = D / 16;  // k-steps of the QK^T product
  constexpr int DB = D / 32;  // 32-row blocks of O^T

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
  const int wave = threadIdx.x >> 6;
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
  float m = -INFINITY, l = 0.f;
  const float c = a.scale * kLog2e;

  u32x4_t kr[D / 32], vr[4];
  if (n_tiles > 0) {
    load_tile<D>(kg, vg, 0, a.Nk, kr, vr);
    store_tile<D>(sm, 0, kr, vr);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile<D>(kg, vg, (t + 1) * kBN, a.Nk, kr, vr);

    // S^T for keys [64t, 64t+64) x this wave's 32 queries: two 32x32 blocks.
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      const int row = kb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(&sm.k[buf][row * D + k_swz<D>(row, ks * 2 + hl) * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    if (t >= n_clean) {  // tile crosses the diagonal or the key tail
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * kBN + kb * 32 + (r / 4) * 8 + hl * 4 + (r % 4);
          const bool vis = key < a.Nk && (!a.causal || key <= qrow + off);
          if (!vis) sacc[kb][r] = -INFINITY;
        }
    }

    // running max of this query row (both halves of the wave)
    float mx = sacc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
    mx = halves_max(mx) * c;
    const float mn = fmaxf(m, mx);
    const float mu = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - mu);
    m = mn;

    float psum = 0.f;
    bf16x8_t pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(sacc[kb][r], c, -mu));
        psum += p[r];
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(p[half * 8 + 2 * i], p[half * 8 + 2 * i + 1]);
        pf[kb * 2 + half] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

    // O^T += V^T P^T over the 64 keys, four k-steps of 16
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 32 + col;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(&sm.vt[buf][((kk * 4 + hl) * D + d) * 4]);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(&sm.vt[buf][((kk * 4 + 2 + hl) * D + d) * 4]);
        const u32x4_t va = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pf[kk], oacc[db], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) store_tile<D>(sm, buf ^ 1, kr, vr);
    __syncthreads();
  }

  // ---- epilogue: one division, bf16 output, natural-log LSE
  const float lt = halves_sum(l);
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
