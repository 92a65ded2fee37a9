// Single-token decode against a contiguous or paged KV cache: split-K partial
// kernel plus a log-sum-exp merge kernel.
//
// What is computed: one new query per (sequence, query head) against every
// cached key of the sequence, the new token included, no mask ("Генерация и
// KV-кэш", section "KV-кэш для одной головы на NumPy") — or, with a sliding
// window of W keys, against the last W only ("Module 09: Efficient
// Attention", section "Attention Mask Gallery"); query head h reads KV
// head floor(h / n_rep) ("Module 09: Efficient Attention", "The Math: Sharing
// Keys and Values"); paged token t sits at (block_table[t / bs], t % bs) of a
// (num_blocks, bs, Hkv, d) pool ("Module 09", "Code: A Paged KV Cache from
// Scratch").
//
// Decode reads every cached byte once and does 4 flop per byte of bf16 cache,
// so it is bound by HBM bandwidth.  The design is about streaming:
//   * a workgroup owns (sequence b, KV head g, a group of QH query heads of g,
//     split s) and reads split s of g's keys and values exactly once for all
//     QH heads;
//   * a token row (d elements) is read by G = d/16 lanes, 16 elements each, as
//     16-byte loads; a wave covers 64/G tokens per load and issues U such loads
//     for K and for V before using any of them (U = 2; 4 for FP8, whose rows
//     are half as long, so that as many bytes are in flight per wave: measured
//     on MI355X, the paged FP8 batch 808 -> 781 us);
//   * the cache is read with non-temporal loads: each byte is used once per
//     call, and without the hint the stream fills L2 with lines that are never
//     read again (measured on MI355X: the contiguous B = 64 batch 229 -> 201 us,
//     the paged B = 128 batch 1515 -> 1403 us);
//   * bf16: q.k with v_dot2_f32_bf16; the weighted sum of V pairs the two
//     tokens a lane holds per stage and uses v_dot2 as well (the weights go to
//     bf16 there, as in prefill; the row sum stays fp32);
//   * scores are reduced across the G lanes with DPP, and each G-lane group
//     keeps its own running (max, sum, output) — the recurrence of the "Li
//     Hongyi, Machine Learning 2026" notes, lecture "FlashAttention" — so the
//     loop has no cross-group traffic; the groups, then the four waves, are
//     combined once at the end;
//   * when a sequence spans several splits, a one-workgroup kernel first
//     lists the (sequence, split) work items longest first, and the split
//     kernel's workgroups take them in that order;
//   * the partial (normalised output, log-sum-exp) of each split goes to the
//     workspace and a last kernel merges a sequence's splits with weights
//     exp(lse_s - max lse) — the same recurrence applied to whole splits.  A
//     sequence that fits in one split is written directly.
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kElems = 16;     // elements of a row held by one lane
constexpr float kSlack = 8.f;  // log2 units a running max may lag before rescaling

// Cache element types: float, uint16_t (bf16) and uint8_t (FP8 E4M3 codes).
// Queries and outputs are fp32 with an fp32 cache and bf16 otherwise.
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kVecs = 4, kQVecs = 4, kU = 2; };     // 16 floats = 4 x 16 B
template <> struct Elem<uint16_t> { static constexpr int kVecs = 2, kQVecs = 2, kU = 2; };  // 16 bf16  = 2 x 16 B
template <> struct Elem<uint8_t> { static constexpr int kVecs = 1, kQVecs = 2, kU = 4; };   // 16 codes = 16 B (q: bf16)

// Two E4M3 codes (the low or the high half of w) as two bf16, exactly (a code
// has 3 mantissa bits and an exponent well inside bf16's range).
template <bool HIGH>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
}

// Partial dot product of a lane's 16 elements of q and k.
__device__ __forceinline__ float dot16(const u32x4_t* q, const u32x4_t* k, float) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = fmaf(__uint_as_float(q[j][t]), __uint_as_float(k[j][t]), acc);
  return acc;
}
__device__ __forceinline__ float dot16(const u32x4_t* q, const u32x4_t* k, uint16_t) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[j][t]), as_bf16x2(k[j][t]), acc, false);
  return acc;
}

// q (16 bf16: elements 2t, 2t+1 in dword t) . k (16 E4M3 codes, 4 per dword)
__device__ __forceinline__ float dot16(const u32x4_t* q, const u32x4_t* k, uint8_t) {
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[(2 * t) / 4][(2 * t) % 4]), fp8x2_to_bf16x2<false>(k[0][t]),
                                          acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[(2 * t + 1) / 4][(2 * t + 1) % 4]),
                                          fp8x2_to_bf16x2<true>(k[0][t]), acc, false);
  }
  return acc;
}

// o[0..15] += p * v (the lane's 16 elements, in the lane's element order).
__device__ __forceinline__ void axpy16(float* o, float p, const u32x4_t* v, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) o[j * 4 + t] = fmaf(p, __uint_as_float(v[j][t]), o[j * 4 + t]);
}
__device__ __forceinline__ void axpy16(float* o, float p, const u32x4_t* v, uint16_t) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[j * 8 + 2 * t] = fmaf(p, bf16lo_to_f32(v[j][t]), o[j * 8 + 2 * t]);
      o[j * 8 + 2 * t + 1] = fmaf(p, bf16hi_to_f32(v[j][t]), o[j * 8 + 2 * t + 1]);
    }
}

// Index in the d-vector of element i (0..15) held by lane `sub` of a G-lane group.
template <typename T, int G>
__device__ __forceinline__ int elem_index(int sub, int i) {
  constexpr int per = 16 / (int)sizeof(T);         // elements per 16-byte vector
  return ((i / per) * G + sub) * per + (i % per);
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (G == 8) x += dpp<kDppHalfMirror>(x);
  return x;
}

// Compiler-only fences (they emit no instruction): memory operations may not
// move across the asm, and the machine scheduler may not move anything across
// the sched_barrier.  Together they keep the prefetch loads of the next stage
// ahead of the current stage's arithmetic; without them the loads are sunk next
// to their first use and the pipeline collapses.
__device__ __forceinline__ void keep_loads_here() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Keys [kbeg, L) of a sequence of L cached tokens: all of them, or the last
// `window` with a sliding window.  They are cut into splits of `chunk` tokens
// counted from kbeg.  An invalid length gets one split, which reports it.
struct KeyRange {
  int kbeg, ns;
  bool bad;
};
__device__ __forceinline__ KeyRange key_range(int L, const DecodeArgs& a) {
  KeyRange r;
  r.bad = L < 0 || L > a.max_seq_len;
  r.kbeg = (!r.bad && a.window > 0) ? max(0, L - a.window) : 0;
  const int n = r.bad ? 0 : L - r.kbeg;
  r.ns = n <= a.split_tokens ? 1 : (n + a.split_tokens - 1) / a.split_tokens;
  return r;
}

// Combine running state (m, l, o) with (m2, l2, o2); m are log2-domain maxima.
template <int N>
__device__ __forceinline__ void combine(float& m, float& l, float* o, float m2, float l2, const float* o2) {
  const float mn = fmaxf(m, m2);
  const float a1 = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
  const float a2 = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = mn;
}

// One workgroup: the (sequence, split) work items sorted by length, longest
// first, into a.plan (a counting sort over 64-token buckets; the order among
// equal lengths is free, and no result depends on it).  The split kernel's
// workgroups take the items in this order and the hardware starts them in
// order as slots free up, so the short last splits of the sequences run at
// the end instead of leaving slots idle behind a long one (list scheduling,
// longest first).  plan[0] = number of items.
constexpr int kPlanTokens = 64;
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
  __shared__ int cnt[kPlanBuckets];
  for (int i = threadIdx.x; i < kPlanBuckets; i += kPlanThreads) cnt[i] = 0;
  __syncthreads();
  auto bucket = [&](int L, const KeyRange& kr, int s) {
    if (kr.bad) return 0;
    const int t0 = kr.kbeg + s * a.split_tokens, t1 = min(L, t0 + a.split_tokens);
    return min(kPlanBuckets - 1, (t1 - t0 + kPlanTokens - 1) / kPlanTokens);
  };
  for (int b = threadIdx.x; b < a.B; b += kPlanThreads) {
    const int L = a.seq_lens[b];
    const KeyRange kr = key_range(L, a);
    for (int s = 0; s < kr.ns; ++s) atomicAdd(&cnt[kPlanBuckets - 1 - bucket(L, kr, s)], 1);
  }
  __syncthreads();
  const int total = plan_exclusive_scan(cnt);
  if (threadIdx.x == 0) a.plan[0] = total;
  for (int b = threadIdx.x; b < a.B; b += kPlanThreads) {
    const int L = a.seq_lens[b];
    const KeyRange kr = key_range(L, a);
    for (int s = 0; s < kr.ns; ++s) {
      const int pos = atomicAdd(&cnt[kPlanBuckets - 1 - bucket(L, kr, s)], 1);
      a.plan[1 + pos] = b * a.max_splits + s;
    }
  }
}

template <typename T, int D, int QH, bool PAGED>
__global__ __launch_bounds__(kWaves * 64) void decode_split_kernel(DecodeArgs a) {
  constexpr int G = D / kElems;         // lanes per token row
  constexpr int TPW = 64 / G;           // tokens per wave per load
  constexpr int NV = Elem<T>::kVecs;    // 16-byte vectors per lane per row
  constexpr int QV = Elem<T>::kQVecs;   // 16-byte vectors of a query per lane
  using TQ = typename std::conditional<sizeof(T) == 4, float, uint16_t>::type;  // query / output type
  constexpr int kU = Elem<T>::kU;       // token loads per lane per pipeline stage
  constexpr int TOK_IT = TPW * kU;      // tokens per wave per iteration

  __shared__ float red_o[kWaves][QH][D];
  __shared__ float red_ml[kWaves][QH][2];
  __shared__ int red_bad[kWaves];

  // grid: the (KV head, query-head group) fastest, so the workgroups of all
  // heads of one split are dispatched together and read the same pool blocks
  // (each block interleaves the Hkv heads token by token); then the work item:
  // with several splits, item i of the longest-first list, else x = heads,
  // z = b.
  const int nqg = (a.Hq / a.Hkv) / QH;
  int s, b, gx;
  if (a.plan) {
    const int ngroups = a.Hkv * nqg;
    const int idx = blockIdx.x / ngroups;
    gx = blockIdx.x - idx * ngroups;
    if (idx >= a.plan[0]) return;
    const int item = a.plan[1 + idx];
    b = item / a.max_splits;
    s = item - b * a.max_splits;
  } else {
    gx = blockIdx.x;
    s = 0;
    b = blockIdx.z;
  }
  const int g = gx / nqg;
  const int h0 = g * (a.Hq / a.Hkv) + (gx % nqg) * QH;

  const int L = a.seq_lens[b];
  const KeyRange kr = key_range(L, a);
  const int ns = kr.ns;
  if (s >= ns) return;
  bool bad = kr.bad;
  const int t_begin = bad ? 0 : kr.kbeg + s * a.split_tokens;
  const int t_end = bad ? 0 : min(L, t_begin + a.split_tokens);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int grp = lane / G;
  const int sub = lane % G;
  const float c = a.scale * a.k_scale * kLog2e;

  // this lane's 16 elements of each query head (the elements of the cache
  // vectors it loads: interleaved vectors for fp32/bf16, 16 consecutive
  // elements for FP8)
  u32x4_t q[QH][QV];
  {
    const u32x4_t* qv = reinterpret_cast<const u32x4_t*>(reinterpret_cast<const TQ*>(a.q) + ((size_t)b * a.Hq + h0) * D);
#pragma unroll
    for (int r = 0; r < QH; ++r)
#pragma unroll
      for (int j = 0; j < QV; ++j)
        q[r][j] = qv[r * (D * sizeof(TQ) / 16) + (sizeof(T) == 1 ? sub * QV + j : j * G + sub)];
  }

  float m[QH], l[QH], o[QH][kElems];
#pragma unroll
  for (int r = 0; r < QH; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < kElems; ++i) o[r][i] = 0.f;
  }

  const size_t row_vecs = D * sizeof(T) / 16;  // 16-byte vectors per token row
  const u32x4_t* kbase = reinterpret_cast<const u32x4_t*>(a.k);
  const u32x4_t* vbase = reinterpret_cast<const u32x4_t*>(a.v);
  const int32_t* table = PAGED ? a.block_table + (size_t)b * a.max_blocks_per_seq : nullptr;
  const size_t contig_base = ((size_t)b * a.Hkv + g) * (size_t)a.kv_capacity;

  // Two-stage software pipeline per wave.  Stage n: fetch the block-table
  // entries of iteration n+2, issue the K/V loads of iteration n+1 (their
  // table entries arrived during stage n-1), then compute iteration n.  Loads
  // are never predicated: a lane past the end of the split reads the split's
  // last (valid, finite) row and its score is masked to -inf, so its weight is
  // exactly 0.  Program order keeps the K/V loads of n+1 in flight while
  // iteration n is computed (vmcnt is counted in issue order).
  const int stride = kWaves * TOK_IT;
  struct Buf { u32x4_t k[kU][NV], v[kU][NV]; };

  auto fetch_table = [&](int (&ph)[kU], int t0) {
    if constexpr (PAGED) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int tok = min(t0 + u * TPW + grp, t_end - 1);
        ph[u] = table[tok >> a.log2_block_size];
      }
    }
  };
  auto issue = [&](Buf& B, int t0, const int (&ph)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int tok = min(t0 + u * TPW + grp, t_end - 1);
      size_t row;
      if constexpr (PAGED) {
        int phys = ph[u];
        if (phys < 0 || phys >= a.kv_capacity) { bad = true; phys = 0; }
        row = ((size_t)phys * a.block_size + (tok & (a.block_size - 1))) * a.Hkv + g;
      } else {
        row = contig_base + tok;
      }
      const size_t base = row * row_vecs + sub;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        B.k[u][j] = __builtin_nontemporal_load(&kbase[base + j * G]);
        B.v[u][j] = __builtin_nontemporal_load(&vbase[base + j * G]);
      }
    }
  };
  auto compute = [&](const Buf& B, int t0) {
    // bf16 / FP8: element i of tokens 2p and 2p + 1 of this stage, paired
    // for v_dot2 (token 2p in the low half)
    constexpr int NP = kU / 2;
    uint32_t vpair[NP][kElems];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            vpair[p][j * 8 + 2 * t] = __builtin_amdgcn_perm(B.v[2 * p + 1][j][t], B.v[2 * p][j][t], 0x05040100u);
            vpair[p][j * 8 + 2 * t + 1] = __builtin_amdgcn_perm(B.v[2 * p + 1][j][t], B.v[2 * p][j][t], 0x07060302u);
          }
    } else if constexpr (sizeof(T) == 1) {
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // bytes (tok0[4t], tok1[4t], tok0[4t+1], tok1[4t+1]) and the next two
          const uint32_t lo = __builtin_amdgcn_perm(B.v[2 * p + 1][0][t], B.v[2 * p][0][t], 0x05010400u);
          const uint32_t hi = __builtin_amdgcn_perm(B.v[2 * p + 1][0][t], B.v[2 * p][0][t], 0x07030602u);
          vpair[p][4 * t] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(lo));
          vpair[p][4 * t + 1] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(lo));
          vpair[p][4 * t + 2] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<false>(hi));
          vpair[p][4 * t + 3] = __builtin_bit_cast(uint32_t, fp8x2_to_bf16x2<true>(hi));
        }
    }
#pragma unroll
    for (int r = 0; r < QH; ++r) {
      float sc[kU];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float part = group_sum<G>(dot16(q[r], B.k[u], T{}));
        sc[u] = (t0 + u * TPW + grp < t_end) ? part * c : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      // Rescale only when some lane's max grows by more than kSlack: the
      // state (m, l, o) stays exact for any reference m >= the true max - kSlack,
      // the weights are then at most 2^kSlack, and most stages skip the multiply.
      const float mn = fmaxf(m[r], mx);
      if (__any(mn > m[r] + kSlack)) {
        const float alpha = fast_exp2(m[r] - ((mn == -INFINITY) ? 0.f : mn));
        l[r] *= alpha;
#pragma unroll
        for (int i = 0; i < kElems; ++i) o[r][i] *= alpha;
        m[r] = mn;
      }
      const float mu = (m[r] == -INFINITY) ? 0.f : m[r];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        sc[u] = fast_exp2(sc[u] - mu);
        psum += sc[u];
      }
      l[r] += psum;
      if constexpr (sizeof(T) <= 2) {
        // o += p0 V0 + p1 V1 for all 16 elements with one v_dot2 each, per pair
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const bf16x2_t pw = as_bf16x2(pack_bf16x2(sc[2 * p], sc[2 * p + 1]));
#pragma unroll
          for (int i = 0; i < kElems; ++i)
            o[r][i] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(vpair[p][i]), pw, o[r][i], false);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) axpy16(o[r], sc[u], B.v[u], T{});
      }
    }
  };

  int t0 = t_begin + wave * TOK_IT;
  if (t0 < t_end) {
    Buf A, Bb;
    int pA[kU], pB[kU];
    fetch_table(pA, t0);
    fetch_table(pB, t0 + stride);
    issue(A, t0, pA);
    // No branch around the prefetch: past the end of the split every lane's
    // token is clamped to the split's last row, so the one surplus stage per
    // wave re-reads a single cached row.
    for (;;) {
      fetch_table(pA, t0 + 2 * stride);
      issue(Bb, t0 + stride, pB);
      keep_loads_here();
      compute(A, t0);
      if (t0 + stride >= t_end) break;
      fetch_table(pB, t0 + 3 * stride);
      issue(A, t0 + 2 * stride, pA);
      keep_loads_here();
      compute(Bb, t0 + stride);
      if (t0 + 2 * stride >= t_end) break;
      t0 += 2 * stride;
    }
  }

  // combine the TPW groups of this wave (lanes with equal `sub`)
#pragma unroll
  for (int x = G; x < 64; x <<= 1) {
#pragma unroll
    for (int r = 0; r < QH; ++r) {
      float o2[kElems];
#pragma unroll
      for (int i = 0; i < kElems; ++i) o2[i] = __shfl_xor(o[r][i], x);
      const float m2 = __shfl_xor(m[r], x);
      const float l2 = __shfl_xor(l[r], x);
      combine<kElems>(m[r], l[r], o[r], m2, l2, o2);
    }
  }
  const bool wave_bad = __any(bad);
  if (lane < G) {
#pragma unroll
    for (int r = 0; r < QH; ++r) {
#pragma unroll
      for (int i = 0; i < kElems; ++i) red_o[wave][r][elem_index<T, G>(sub, i)] = o[r][i];
      if (sub == 0) {
        red_ml[wave][r][0] = m[r];
        red_ml[wave][r][1] = l[r];
      }
    }
  }
  if (lane == 0) red_bad[wave] = wave_bad;
  __syncthreads();

  const bool any_bad = red_bad[0] | red_bad[1] | red_bad[2] | red_bad[3];
  for (int idx = threadIdx.x; idx < QH * D; idx += kWaves * 64) {
    const int r = idx / D, e = idx % D;
    float mm = red_ml[0][r][0], ll = red_ml[0][r][1], oo = red_o[0][r][e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) combine<1>(mm, ll, &oo, red_ml[w][r][0], red_ml[w][r][1], &red_o[w][r][e]);
    const int h = h0 + r;
    float out = ll > 0.f ? oo / ll * a.v_scale : 0.f;
    float lse = ll > 0.f ? (mm + fast_log2(ll)) * kLn2 : -INFINITY;
    if (any_bad) out = lse = NAN;
    if (ns == 1) {
      if constexpr (sizeof(T) == 4) {
        reinterpret_cast<float*>(a.o)[((size_t)b * a.Hq + h) * D + e] = out;
      } else {
        const uint32_t pk = pack_bf16x2(out, 0.f);
        reinterpret_cast<uint16_t*>(a.o)[((size_t)b * a.Hq + h) * D + e] = (uint16_t)(pk & 0xffffu);
      }
      if (a.lse && e == 0) a.lse[(size_t)b * a.Hq + h] = lse;
    } else {
      const size_t slot = ((size_t)b * a.Hq + h) * a.max_splits + s;
      a.ws_o[slot * D + e] = out;
      if (e == 0) a.ws_lse[slot] = lse;
    }
  }
}

// One wave per (sequence, query head): the lanes first share out the split
// log-sum-exps (max, then weights and their sum, reduced across the wave),
// then each lane sums its d/64 output elements over the splits with
// independent loads.  Four (sequence, head) rows per workgroup.
constexpr int kMergeRows = 4;
template <typename T, int D>
__global__ __launch_bounds__(64 * kMergeRows) void decode_merge_kernel(DecodeArgs a) {
  constexpr int E = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * kMergeRows + (threadIdx.x >> 6);
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  const int ns = key_range(a.seq_lens[b], a).ns;
  if (ns == 1) return;  // written by the split kernel
  const size_t slot0 = (size_t)bh * a.max_splits;
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, a.ws_lse[slot0 + s]);
  for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
  float wsum = 0.f;
  for (int s = lane; s < ns; s += 64) wsum += __expf(a.ws_lse[slot0 + s] - M);
  for (int x = 32; x >= 1; x >>= 1) wsum += __shfl_xor(wsum, x);
  float acc[E];
#pragma unroll
  for (int j = 0; j < E; ++j) acc[j] = 0.f;
  const float* wo = a.ws_o + slot0 * D + lane * E;
#pragma unroll 4
  for (int s = 0; s < ns; ++s) {
    const float w = __expf(a.ws_lse[slot0 + s] - M);
#pragma unroll
    for (int j = 0; j < E; ++j) acc[j] = fmaf(w, wo[(size_t)s * D + j], acc[j]);
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const float out = acc[j] * inv;
    if constexpr (sizeof(T) == 4) {
      reinterpret_cast<float*>(a.o)[(size_t)bh * D + lane * E + j] = out;
    } else {
      reinterpret_cast<uint16_t*>(a.o)[(size_t)bh * D + lane * E + j] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xffffu);
    }
  }
  if (a.lse && lane == 0) a.lse[bh] = M + __logf(wsum);
}

template <typename T, int D, int QH>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t st) {
  const int nqg = (a.Hq / a.Hkv) / QH;
  dim3 grid(a.Hkv * nqg, 1, a.B);
  if (a.max_splits > 1) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
    grid = dim3((unsigned)((long long)a.Hkv * nqg * a.B * a.max_splits), 1, 1);
  }
  if (a.block_table)
    hipLaunchKernelGGL((decode_split_kernel<T, D, QH, true>), grid, dim3(kWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, QH, false>), grid, dim3(kWaves * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((a.B * a.Hq + kMergeRows - 1) / kMergeRows), dim3(64 * kMergeRows),
                     0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
  const int n_rep = a.Hq / a.Hkv;
  if (n_rep % 8 == 0) return launch_typed<T, D, 8>(a, st);
  if (n_rep % 4 == 0) return launch_typed<T, D, 4>(a, st);
  if (n_rep % 2 == 0) return launch_typed<T, D, 2>(a, st);
  return launch_typed<T, D, 1>(a, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, KvType t, hipStream_t st) {
  switch (t) {
    case KvType::BF16: return a.d == 64 ? launch_d<uint16_t, 64>(a, st) : launch_d<uint16_t, 128>(a, st);
    case KvType::FP8: return a.d == 64 ? launch_d<uint8_t, 64>(a, st) : launch_d<uint8_t, 128>(a, st);
    default: return a.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
  }
}

}  // namespace fa
