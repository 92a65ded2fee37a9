// fp32 prefill: exact attention with the streaming softmax, fp32 throughout.
//
// Tiling follows the outer-loop-over-query-tiles / inner-loop-over-key-tiles
// scheme of "KV Cache, Flash Attention and Inference Optimization", section
// "the tiling trick"; the per-row update is the running max / running sum
// recurrence of the "Li Hongyi, Machine Learning 2026" notes (lecture
// "FlashAttention"), in the unnormalised-accumulator form of the same lesson's
// "tiled softmax" step: the accumulator and the sum are both multiplied by
// exp(m_old - m_new) when the max grows, and divided once at the end.
//
// One wave (64 lanes) owns 64 query rows, one row per lane: the row's query and
// output live in registers and every key/value tile is read from LDS as a
// broadcast.  This is the precision path (fp32 in/out); the bf16 path uses the
// MFMA kernel.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one per lane)
constexpr int kKeys = 32;   // keys per LDS tile
constexpr int kSub = 8;     // keys per softmax update

template <int D, bool PAGED>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  __shared__ float4 Ks[kKeys * D / 4];
  __shared__ float4 Vs[kKeys * D / 4];

  const int lane = threadIdx.x;
  const int nqb = (a.Nq + kRows - 1) / kRows;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int h = bh % a.Hq;
  const int b = bh / a.Hq;
  const int g = h / (a.Hq / a.Hkv);

  const int row = qb * kRows + lane;
  const bool row_ok = row < a.Nq;

  // Keys: Nk per head, or the cached length of sequence b (its newest Nq
  // tokens being the queries).  A length outside the contract or a block id
  // outside the pool turns the rows into NaN.
  int Nk = a.Nk;
  size_t head_rows = (size_t)a.Nk;
  bool bad = false;
  if (a.seq_lens) {
    Nk = a.seq_lens[b];
    head_rows = (size_t)a.kv_capacity;
    bad = Nk < 0 || Nk > a.max_seq_len || (a.causal && Nk < a.Nq);
    if (bad) Nk = 0;
  }
  const int off = Nk - a.Nq;
  // keys [lo, lim) are visible to this row (lo > 0 only with a sliding window)
  const int lim = a.causal ? min(Nk, row + off + 1) : Nk;
  const int lo = a.window > 0 ? row + off - a.window + 1 : 0;
  const int last_row = min(a.Nq, (qb + 1) * kRows) - 1;
  int kend = a.causal ? min(Nk, last_row + off + 1) : Nk;
  if (bad) kend = 0;
  // first key any row of the workgroup sees, and the tile it falls in; keys
  // before klo are never read (their blocks may have been released)
  const int klo = a.window > 0 ? max(0, qb * kRows + off - a.window + 1) : 0;
  const int kbeg = (klo / kKeys) * kKeys;
  const int32_t* trow = PAGED ? a.block_table + (size_t)b * a.max_blocks_per_seq : nullptr;
  if (PAGED && kend > kbeg) {
    const int ntok = min(((kend + kKeys - 1) / kKeys) * kKeys, Nk);  // rows the staging loop reads
    const int ne = (ntok + a.block_size - 1) >> a.log2_block_size;
    int oob = 0;
    for (int i = (klo >> a.log2_block_size) + lane; i < ne; i += 64) {
      const int e = trow[i];
      oob |= (e < 0) | (e >= a.kv_capacity);
    }
    if (__syncthreads_or(oob)) {
      bad = true;
      kend = 0;
    }
  }

  const float c = a.scale * kLog2e;  // scores kept in log2 units
  const float* qp = reinterpret_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq + min(row, a.Nq - 1)) * D;
  // first element of key/value row j of this head
  auto kv_row = [&](const void* base, int j) -> const float4* {
    const float* p = reinterpret_cast<const float*>(base);
    if constexpr (PAGED) {
      const int e = trow[j >> a.log2_block_size];
      return reinterpret_cast<const float4*>(
          p + (((size_t)e * a.block_size + (j & (a.block_size - 1))) * a.Hkv + g) * D);
    } else {
      return reinterpret_cast<const float4*>(p + ((size_t)(b * a.Hkv + g) * head_rows + j) * D);
    }
  };

  float qr[D];
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    float4 t = *reinterpret_cast<const float4*>(qp + e);
    qr[e] = t.x * c; qr[e + 1] = t.y * c; qr[e + 2] = t.z * c; qr[e + 3] = t.w * c;
  }
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += kKeys) {
    // stage K and V rows [k0, k0 + kKeys) (zeros outside [klo, Nk))
    for (int i = lane; i < kKeys * D / 4; i += 64) {
      const int r = i / (D / 4), cc = i % (D / 4);
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (k0 + r < Nk && k0 + r >= klo) {
        kv = kv_row(a.k, k0 + r)[cc];
        vv = kv_row(a.v, k0 + r)[cc];
      }
      Ks[i] = kv;
      Vs[i] = vv;
    }
    __syncthreads();
    for (int j0 = 0; j0 < kKeys; j0 += kSub) {
      float s[kSub];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < D; e += 4) {
          float4 kk = Ks[(j0 + j) * (D / 4) + e / 4];
          dot = fmaf(qr[e], kk.x, dot);
          dot = fmaf(qr[e + 1], kk.y, dot);
          dot = fmaf(qr[e + 2], kk.z, dot);
          dot = fmaf(qr[e + 3], kk.w, dot);
        }
        s[j] = (k0 + j0 + j < lim && k0 + j0 + j >= lo) ? dot : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      if (m_new == -INFINITY) continue;  // nothing visible yet in this row
      const float alpha = fast_exp2(m - m_new);  // 0 while m is -inf
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        s[j] = fast_exp2(s[j] - m_new);
        psum += s[j];
      }
      l = l * alpha + psum;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        float o0 = acc[e] * alpha, o1 = acc[e + 1] * alpha, o2 = acc[e + 2] * alpha, o3 = acc[e + 3] * alpha;
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
          float4 vv = Vs[(j0 + j) * (D / 4) + e / 4];
          o0 = fmaf(s[j], vv.x, o0);
          o1 = fmaf(s[j], vv.y, o1);
          o2 = fmaf(s[j], vv.z, o2);
          o3 = fmaf(s[j], vv.w, o3);
        }
        acc[e] = o0; acc[e + 1] = o1; acc[e + 2] = o2; acc[e + 3] = o3;
      }
      m = m_new;
    }
    __syncthreads();
  }

  if (!row_ok) return;
  const float inv = bad ? __builtin_nanf("") : l > 0.f ? 1.f / l : 0.f;
  float* op = reinterpret_cast<float*>(a.o) + ((size_t)(b * a.Hq + h) * a.Nq + row) * D;
#pragma unroll
  for (int e = 0; e < D; e += 4)
    *reinterpret_cast<float4*>(op + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  if (a.lse)
    a.lse[(size_t)(b * a.Hq + h) * a.Nq + row] = bad ? __builtin_nanf("") : l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  const int nqb = (a.Nq + kRows - 1) / kRows;
  const long long grid = (long long)nqb * a.Hq * a.B;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool paged = a.block_table != nullptr;
  if (a.d == 64) {
    if (paged) hipLaunchKernelGGL((prefill_f32_kernel<64, true>), dim3((unsigned)grid), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<64, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  } else {
    if (paged) hipLaunchKernelGGL((prefill_f32_kernel<128, true>), dim3((unsigned)grid), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((prefill_f32_kernel<128, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fa
