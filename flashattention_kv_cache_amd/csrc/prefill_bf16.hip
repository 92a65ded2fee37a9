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
//   * workgroup = 8 waves = 256 query rows, one workgroup per CU (two waves
//     per SIMD); each wave owns 32 rows.  The rows are 256 / hw consecutive
//     positions of hw query heads that read the same KV head (hw = the
//     largest power of two dividing Hq / Hkv, at most 8): every K/V tile
//     still feeds 256 rows, while a query tile spans fewer positions, so the
//     causal diagonal crosses fewer key tiles (one instead of four at
//     Hq / Hkv = 4; measured on MI355X at N = 4096: 2.8% less time than 256
//     positions of one head, same bits).  Both waves of a SIMD belong to the
//     same workgroup, so neither can starve the other (two co-resident
//     workgroups were measured to progress at rates ~1.4x apart, leaving each
//     CU's last stretch to a single workgroup).  Key and
//     value tiles of 64 rows go from HBM straight into LDS with
//     global_load_lds_dwordx4 (no staging registers, no vector ALU work),
//     issued from inline assembly so that nothing waits for them before the
//     end of the tile they overlap:
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
//     the source addresses of the direct loads) so that both the 16-byte K
//     operand reads and the transposed V reads are free of bank conflicts.
//   * software pipeline inside each wave: stage t runs the QK^T MFMAs of tile
//     t+1 and the PV MFMAs of tile t-1 interleaved with the softmax arithmetic
//     of tile t (all three are independent), so each wave keeps its matrix
//     cores fed while its vector ALUs work; the direct loads of K(t+2) and
//     V(t) fly during the whole stage.  One barrier per tile.
//   * causal: only key tiles left of and on the diagonal are visited, the mask
//     is evaluated only on tiles that cross the diagonal or the key tail, and
//     a workgroup runs two query tiles, qb and nqb - 1 - qb, whose key-tile
//     counts add up to the same total for every pair, so all workgroups of a
//     launch carry equal work; workgroups that share a KV head are placed on
//     the same XCD (dispatch is round-robin over the 8 XCDs) so that head's
//     K/V stays in that XCD's L2.  On the diagonal, a wave stops its
//     products at the first key tile that all of its 32 rows mask (their
//     weights would be exact zeros) and from there on only copies its share
//     of the tiles and meets the barriers.
//   * the output tile leaves through LDS (the K/V tiles are free by then), so
//     that each global store writes 1 KiB of consecutive rows.
//   * the weights of a tile are taken against the running max as it stands,
//     without a pass over the tile's scores first: (m, l, O) is exact for
//     any reference m, and what the reference must keep in check is the size
//     of the weights.  A lane whose sum of the tile's weights exceeds
//     2^kSlack (as any weight above 2^kSlack makes it) sends the wave back
//     over the tile: S(t) again from K(t), read from global memory since its
//     LDS buffer is being refilled, then its exact max, the rescale and new
//     weights.  Only a wave's first tile takes its max first.  This removes
//     the max's ~30 vector instructions per stage, which at the clock the
//     matrix cores' power allows cost time as vector work.  With a sliding
//     window, whose rows find their first keys tiles apart, the max still
//     comes first.
//   * the row sum is accumulated in fp32 from the unrounded weights (a sum of
//     the bf16-rounded weights would move the log-sum-exp by ~1e-3 on short
//     rows).
#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;              // waves per workgroup, 32 query rows each
constexpr int kBM = 32 * kWaves;        // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 64 * kWaves;
constexpr int kCopyRows = kBN / kWaves;  // tile rows one wave copies
constexpr float kSlack = 8.f;  // log2 units a running max may lag before rescaling
constexpr float kSumMax = 256.f;  // 2^kSlack: largest accepted sum of a lane's weights of one tile

template <int D>
struct Smem {
  union {
    struct {
      uint16_t k[2][kBN * D];  // row-major K tiles, chunks swizzled by row % 8
      uint16_t v[2][kBN * D];  // row-major V tiles, chunks swizzled by 2 * (row % 4)
    };
    uint16_t o[kWaves][32 * D];  // epilogue: each wave's 32 output rows, chunks swizzled as K
  };
};
static_assert(sizeof(Smem<128>) == 4 * kBN * 128 * 2 && sizeof(Smem<64>) == 4 * kBN * 64 * 2, "O staging fits the K/V tiles");

// The LDS has 64 banks of 4 bytes: a 16-byte read is served 16 lanes per
// cycle, an 8-byte read 32 lanes per cycle.  Swizzles are XOR masks on the
// 16-byte chunk index of a row.
//   K operand reads: 16 lanes read 16 consecutive rows at one logical chunk.
//     d=128 (16 chunks per 256-byte row): mask = row % 16.
//     d=64 (8 chunks per 128-byte row, two rows per bank line): mask = (row/2) % 8.
//   V transposed reads: 32 lanes read rows 4i..4i+3 at 4 consecutive chunks.
//     d=128: mask = 4 (row % 4);  d=64: mask = 4 ((row/2) % 2).
template <int D> __device__ __forceinline__ int k_swz(int row) { return (row / (128 / D)) & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int v_swz(int row) { return ((row / (128 / D)) & (D / 32 - 1)) << 2; }

// Per-lane layout of one tile copy: instruction i of this wave fills LDS rows
// (wave * IPW + i) * RPI .. + RPI - 1 of the tile.
template <int D, bool IS_V>
struct TileCopy {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per wave instruction
  static constexpr int IPW = kCopyRows / RPI;  // instructions per wave
  uint32_t off[IPW];                         // byte offset of this lane's chunk within the tile

  __device__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = (wave * IPW + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ (IS_V ? v_swz<D>(row) : k_swz<D>(row));
      off[i] = (uint32_t)((row * D + c * 8) * 2);
    }
  }
  // Rows [key0, key0 + 64) of one head (src = row 0 of the head) into dst.
  // Rows before klo are read from row klo and rows at or past Nk from row
  // Nk - 1 (harmless: those keys get weight 0 and the substituted V rows are
  // finite; rows outside [klo, Nk) are never touched).
  __device__ __forceinline__ void copy(const uint16_t* src, const uint16_t* dst_tile, int key0, int klo, int Nk,
                                       int wave, int lane) const {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u16*)dst_tile + (uint32_t)(wave * IPW * RPI * D * 2);
    if (key0 >= klo && key0 + kBN <= Nk) {
      const uint16_t* base = src + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < IPW; ++i) lds_dma_saddr(off[i], base, lds0 + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int row = (wave * IPW + i) * RPI + lane / CPR;
        const int key = min(max(key0 + row, klo), Nk - 1);
        const int c = (lane % CPR) ^ (IS_V ? v_swz<D>(row) : k_swz<D>(row));
        lds_dma_vaddr(src + (size_t)key * D + c * 8, lds0 + i * 1024);
      }
    }
  }
};

// The same tile copy from a paged pool (num_blocks, block_size, Hkv, D): the
// kCopyRows rows a wave copies are consecutive tokens.  When they sit in one
// block (block_size >= kCopyRows and the tile is not the sequence's last) a wave needs one
// block id and its lanes add fixed offsets to one scalar base; otherwise each
// lane looks up the block of its own row.
template <int D, bool IS_V>
struct PagedCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int IPW = kCopyRows / RPI;
  uint32_t off[IPW];  // byte offset of this lane's chunk from the wave's first token

  __device__ void init(int wave, int lane, uint32_t slot_elems) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int local = i * RPI + lane / CPR;
      const int row = wave * IPW * RPI + local;
      const int c = (lane % CPR) ^ (IS_V ? v_swz<D>(row) : k_swz<D>(row));
      off[i] = (local * slot_elems + c * 8) * 2;
    }
  }
  // Tokens tok0 .. tok0 + kCopyRows - 1 of the sequence, all in physical block
  // blk at slots slot0 .. (pool = slot 0 of block 0 at this KV head).
  __device__ __forceinline__ void fast(const uint16_t* pool, int blk, int slot0, int bs, size_t slot_elems,
                                       const uint16_t* dst_tile, int wave) const {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u16*)dst_tile + (uint32_t)(wave * IPW * RPI * D * 2);
    const uint16_t* base = pool + ((size_t)blk * bs + slot0) * slot_elems;
#pragma unroll
    for (int i = 0; i < IPW; ++i) lds_dma_saddr(off[i], base, lds0 + i * 1024);
  }
  // Any block size, any position: tokens before klo read token klo, tokens at
  // or past Nk read token Nk - 1 (blocks outside [klo, Nk) are never touched).
  __device__ __forceinline__ void slow(const uint16_t* pool, const int32_t* trow, int key0, int klo, int Nk,
                                       int lbs, int bs, size_t slot_elems, const uint16_t* dst_tile, int wave,
                                       int lane) const {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_u16*)dst_tile + (uint32_t)(wave * IPW * RPI * D * 2);
    int blk[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {  // every lookup first: the copies below order memory
      const int tok = min(max(key0 + wave * IPW * RPI + i * RPI + lane / CPR, klo), Nk - 1);
      blk[i] = trow[tok >> lbs];
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int row = wave * IPW * RPI + i * RPI + lane / CPR;
      const int tok = min(max(key0 + row, klo), Nk - 1);
      const int c = (lane % CPR) ^ (IS_V ? v_swz<D>(row) : k_swz<D>(row));
      lds_dma_vaddr(pool + ((size_t)blk[i] * bs + (tok & (bs - 1))) * slot_elems + c * 8, lds0 + i * 1024);
    }
  }
};

// Query heads that share a workgroup: the largest power of two dividing
// n_rep = Hq / Hkv, at most 8.  All of them read the same KV head, and the
// workgroup's 256 rows are 256 / hw consecutive positions of each.
__host__ __device__ __forceinline__ int heads_per_workgroup(int n_rep) {
  const int p = n_rep & -n_rep;
  return p < 8 ? p : 8;
}

// Key tiles that query tile qb (P positions) of sequence b visits (the key
// range run_tile computes): with a cache (seq_lens) the sequences differ in
// length.
__device__ __forceinline__ int tile_count(const PrefillArgs& a, int W, int P, int b, int qb) {
  const int L = a.seq_lens[b];
  if (L < 0 || L > a.max_seq_len || (a.causal && L < a.Nq)) return 0;
  const int off = L - a.Nq, q0 = qb * P, last = min(a.Nq, q0 + P) - 1;
  const int kend = a.causal ? min(L, last + off + 1) : L;
  const int tb = (W > 0 ? max(0, q0 + off - W + 1) : 0) / kBN;
  return max(tb, (kend + kBN - 1) / kBN) - tb;
}

// Longest-first work list of a launch over sequences of different lengths:
// the (sequence, query tile) item of rank r when the B * nqb items are ordered
// by key-tile count, longest first, ties by item index (b * nqb + qb).  Every
// workgroup computes the same order (a histogram of the counts, an exclusive
// prefix over it, then a stable selection inside the bucket of rank r), so
// the workgroups of a launch take every item exactly once.  `scratch` holds
// kLptBuckets + 8 words of LDS; all threads of the workgroup call this.
constexpr int kLptBuckets = 1024;  // counts past the last bucket share it (ordered by index)
__device__ int lpt_item(const PrefillArgs& a, int W, int P, int nqb, int r, uint32_t* scratch) {
  uint32_t* hist = scratch;                  // bucket 0 = the most key tiles
  uint32_t* wsum = scratch + kLptBuckets;    // per-wave totals of a scan (8)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.B * nqb;
  auto bucket = [&](int i) { return kLptBuckets - 1 - min(tile_count(a, W, P, i / nqb, i % nqb), kLptBuckets - 1); };
  for (int i = tid; i < kLptBuckets; i += kThreads) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kThreads) atomicAdd(&hist[bucket(i)], 1u);
  __syncthreads();
  // exclusive prefix over the buckets, two per thread: the bucket holding rank r
  static_assert(kLptBuckets == 2 * kThreads, "two buckets per thread");
  const uint32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
  uint32_t incl = h0 + h1;
  for (int x = 1; x < 64; x <<= 1) {
    const uint32_t y = __shfl_up(incl, x, 64);
    if (lane >= x) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t start = incl - h0 - h1;
  for (int w = 0; w < wv; ++w) start += wsum[w];
  __syncthreads();  // every wave has read wsum
  int kb = -1;
  uint32_t target = 0;
  if ((uint32_t)r >= start && (uint32_t)r < start + h0) { kb = 2 * tid; target = r - start; }
  if ((uint32_t)r >= start + h0 && (uint32_t)r < start + h0 + h1) { kb = 2 * tid + 1; target = r - start - h0; }
  if (kb >= 0) { wsum[0] = kb; wsum[1] = target; }
  __syncthreads();
  const int k = (int)wsum[0];
  const uint32_t tgt = wsum[1];
  __syncthreads();
  // the tgt-th item of bucket k in index order
  uint32_t seen = 0;
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    const int i = c0 + tid;
    const bool f = i < n && bucket(i) == k;
    const unsigned long long m = __ballot(f);
    if (lane == 0) wsum[wv] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = seen;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    uint32_t total = 0;
    for (int w = 0; w < kThreads / 64; ++w) total += wsum[w];
    const uint32_t mine = before + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();  // every wave has read wsum
    if (f && mine == tgt) wsum[8 - 1] = i;  // slot 7: read after the next barrier
    __syncthreads();
    seen += total;
    if (seen > tgt) break;
  }
  const int item = (int)wsum[7];
  __syncthreads();  // the scratch may be overwritten after this
  return item;
}

template <int D, bool PAGED, bool WINDOW>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(PrefillArgs a, int nqb, int lpt) {
  __shared__ Smem<D> sm;
  constexpr int KS = D / 16;   // k-steps of the QK^T product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int VPS = 16 / KS; // softmax values of one 32-key block per QK^T k-step

  // ---- work item: a sequence b, hw query heads h .. h + hw - 1 of one KV
  // head, and query tiles of P = 256 / hw positions.  Sequences of one
  // length (plain prefill, or a single cached sequence): (b, h, pair of query
  // tiles), KV-head-major per XCD.  A
  // workgroup takes query tiles nqb - 1 - pr and pr of one head: with a
  // causal mask their key-tile counts add up to the same total for every
  // pair, so all workgroups carry equal work (the lone middle tile of an odd
  // count comes last).  Cached sequences of different lengths (lpt): one
  // query tile per workgroup, the (sequence, tile) items taken longest first
  // so that the hardware's in-order dispatch onto free CUs balances them; the
  // Hq / hw workgroups of an item are consecutive, each XCD getting whole
  // KV-head groups.
  const int id = blockIdx.x;
  const int n_rep = a.Hq / a.Hkv;
  const int hw = heads_per_workgroup(n_rep);  // query heads per workgroup
  const int lhw = __builtin_ctz(hw);
  const int nw = n_rep >> lhw;                // workgroups per (sequence, KV head, query tile)
  const int P = kBM >> lhw;                   // query positions per tile
  const int GP = a.B * a.Hkv;
  int b, h, pr, single = -1;                  // h: the workgroup's first query head
  if (lpt) {
    const int per_item = a.Hkv * nw;
    const int item = lpt_item(a, WINDOW ? a.window : 0, P, nqb, id / per_item, reinterpret_cast<uint32_t*>(sm.k[0]));
    const int j = id % per_item;
    b = item / nqb;
    single = item % nqb;
    pr = 0;
    h = (j % a.Hkv) * n_rep + (j / a.Hkv) * hw;
  } else if ((GP & 7) == 0) {
    const int xcd = id & 7, j = id >> 3;
    const int per = (GP >> 3) * nw;  // work items per pair rank on one XCD
    const int rest = j % per;
    pr = j / per;
    const int gp = xcd + 8 * (rest / nw);
    b = gp / a.Hkv;
    h = (gp % a.Hkv) * n_rep + (rest % nw) * hw;
  } else {
    const int units = GP * nw;  // workgroups per pair rank
    const int bh = id % units;
    pr = id / units;
    b = bh / (a.Hkv * nw);
    h = (bh % (a.Hkv * nw)) * hw;  // (KV head g, sub-group s) -> first head g * n_rep + s * hw
  }
  // The work item is the same for every lane.  In the longest-first path it
  // comes out of LDS, which the compiler treats as per-lane, so it is made
  // scalar explicitly: the K/V head addresses built from it must sit in
  // scalar registers, where the direct-load assembly takes its base.
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  pr = __builtin_amdgcn_readfirstlane(pr);
  single = __builtin_amdgcn_readfirstlane(single);
  const int g = h / n_rep;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5;   // which half of the wave
  const int col = lane & 31;  // query column within the wave's 32 rows
  // wave w: query head h + w % hw, positions 32 * (w / hw) .. + 31 of the tile
  const int hq = h + (wave & (hw - 1));
  const int pw = (wave >> lhw) * 32;

  // ---- the keys: Nk of them per head, or the cached length of sequence b
  // (the queries being its newest tokens).  A length outside the contract, or
  // a block id outside the pool, turns this workgroup's rows into NaN.
  int Nk = a.Nk;
  size_t head_rows = (size_t)a.Nk;
  bool bad_seq = false;
  if (a.seq_lens) {
    Nk = a.seq_lens[b];
    head_rows = (size_t)a.kv_capacity;
    bad_seq = Nk < 0 || Nk > a.max_seq_len || (a.causal && Nk < a.Nq);
    if (bad_seq) Nk = 0;
  }
  const int off = Nk - a.Nq;
  const int W = WINDOW ? a.window : 0;  // > 0: sliding window (causal only)
  const int32_t* trow = PAGED ? a.block_table + (size_t)b * a.max_blocks_per_seq : nullptr;
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + (PAGED ? (size_t)g * D : (size_t)(b * a.Hkv + g) * head_rows * D);
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + (PAGED ? (size_t)g * D : (size_t)(b * a.Hkv + g) * head_rows * D);

  // One query tile: everything from the key range to the epilogue.
  auto run_tile = [&](const int qb) {
    const int q0 = qb * P;
    bool bad = bad_seq;
    const int last_row = min(a.Nq, q0 + P) - 1;
    int kend = a.causal ? min(Nk, last_row + off + 1) : Nk;
    // first key any row of the workgroup sees (its first row's window start)
    const int kbeg = W > 0 ? max(0, q0 + off - W + 1) : 0;
    if (bad) kend = 0;
    const int tb = kbeg / kBN;                              // first key tile visited
    int te = max(tb, (kend + kBN - 1) / kBN);               // one past the last
    if (PAGED && te > tb) {
      // every token a copy may touch: the visited tiles, clamped to the sequence
      const int ntok = min(te * kBN, Nk);
      const int e0 = kbeg >> a.log2_block_size;  // blocks before the first window are never read
      const int ne = (ntok + a.block_size - 1) >> a.log2_block_size;
      int oob = 0;
      for (int i = e0 + threadIdx.x; i < ne; i += kThreads) {
        const int e = trow[i];
        oob |= (e < 0) | (e >= a.kv_capacity);
      }
      if (__syncthreads_or(oob)) {
        bad = true;
        te = tb;
      }
    }
    // tiles in [n_lo, n_clean) need no mask for any row of the workgroup
    const int n_clean = a.causal ? min((q0 + off + 1) / kBN, Nk / kBN) : Nk / kBN;
    const int n_lo = W > 0 ? (max(0, last_row + off - W + 1) + kBN - 1) / kBN : 0;
    // causal: tiles [tb, te_w) hold a key that some row of this wave sees
    const int te_w = a.causal ? min(te, max(tb, (min(q0 + pw + 31, a.Nq - 1) + off) / kBN + 1)) : te;
    // window: this wave's rows see no key before tile tl_w; when tl > tb the
    // wave skips the products of tiles tb .. tl - 1 (exact zeros) and starts
    // its pipeline at tl
    const int tl_w = W > 0 ? max(0, q0 + pw + off - W + 1) / kBN : tb;
    const int tl = (tl_w > tb && tl_w < te_w) ? tl_w : tb;

    // ---- Q^T operand fragments, kept in registers
    const int qrow = q0 + pw + col;
    bf16x8_t qf[KS];
    {
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)(b * a.Hq + hq) * a.Nq + min(qrow, a.Nq - 1)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16 + hl * 8);
    }

    f32x16_t oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    // m: running max (log2 units, -inf before a row's first key); mref: the
    // reference the weights are taken against (m, or 0 while m is -inf)
    float m = -INFINITY, mref = 0.f, l0 = 0.f, l1 = 0.f;
    const float c = a.scale * kLog2e;

    using KCopy = typename std::conditional<PAGED, PagedCopy<D, false>, TileCopy<D, false>>::type;
    using VCopy = typename std::conditional<PAGED, PagedCopy<D, true>, TileCopy<D, true>>::type;
    KCopy kcp;
    VCopy vcp;
    const size_t slot_elems = (size_t)a.Hkv * D;  // paged: elements between consecutive slots
    const int lbs = a.log2_block_size, bsz = a.block_size;
    const bool one_block = bsz >= kCopyRows;      // paged: the tokens a wave copies share a block
    if constexpr (PAGED) {
      kcp.init(wave, lane, (uint32_t)slot_elems);
      vcp.init(wave, lane, (uint32_t)slot_elems);
    } else {
      kcp.init(wave, lane);
      vcp.init(wave, lane);
    }
    // Block id of the first of the tokens this wave copies from tile t
    // (clamped to the sequence; loaded a stage ahead of its use).
    auto entry = [&](int t) { return trow[min(max(t * kBN + wave * kCopyRows, kbeg), Nk - 1) >> lbs]; };
    int eK = 0, eV = 0;  // paged, one_block: block ids for the next stage's K and V copies
    // Tile t of K or V (buffer dst); e = its block id when one_block.
    auto copy_k = [&](uint16_t* dst, int t, int e) {
      if constexpr (PAGED) {
        const int tok0 = t * kBN + wave * kCopyRows;
        if (one_block && tok0 >= kbeg && tok0 + kCopyRows <= Nk)
          kcp.fast(kg, __builtin_amdgcn_readfirstlane(e), tok0 & (bsz - 1), bsz, slot_elems, dst, wave);
        else
          kcp.slow(kg, trow, t * kBN, kbeg, Nk, lbs, bsz, slot_elems, dst, wave, lane);
      } else {
        kcp.copy(kg, dst, t * kBN, kbeg, Nk, wave, lane);
      }
    };
    auto copy_v = [&](uint16_t* dst, int t, int e) {
      if constexpr (PAGED) {
        const int tok0 = t * kBN + wave * kCopyRows;
        if (one_block && tok0 >= kbeg && tok0 + kCopyRows <= Nk)
          vcp.fast(vg, __builtin_amdgcn_readfirstlane(e), tok0 & (bsz - 1), bsz, slot_elems, dst, wave);
        else
          vcp.slow(vg, trow, t * kBN, kbeg, Nk, lbs, bsz, slot_elems, dst, wave, lane);
      } else {
        vcp.copy(vg, dst, t * kBN, kbeg, Nk, wave, lane);
      }
    };

    // LDS element offset of this lane's K operand (row kb*32 + col, logical
    // 16-byte chunk ks*2 + hl), and of its V^T transposed reads.
    auto k_off = [&](int kb, int ks) {
      const int row = kb * 32 + col;
      return row * D + (((ks * 2 + hl) ^ k_swz<D>(row)) * 8);
    };
    // V^T operand for k-step kk (keys 16kk .. 16kk+15) and dims db*32 .. +31:
    // lane L of 16-lane group gi reads row key(j) = 16kk + 8*half + 4*(gi/2) + j
    // with j = (L%16)/4, at dims db*32 + 16*(gi%2) + 4*(L%4) .. +3; the
    // transpose hands lane L the 4 keys of dim db*32 + L%32.
    const int gi = lane >> 4, li = lane & 15;
    auto v_off = [&](int kk, int half, int db) {
      const int row = kk * 16 + half * 8 + (gi >> 1) * 4 + (li >> 2);
      const int d = db * 32 + (gi & 1) * 16 + (li & 3) * 4;
      return row * D + ((((d >> 3) ^ v_swz<D>(row)) << 3) | (d & 7));
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
    // With a window, keys before the row's window start are masked the same way.
    auto mask = [&](f32x16_t (&sacc)[2], int t) {
      const int base = t * kBN + hl * 4;
      const int lim = (a.causal ? min(qrow + off, Nk - 1) : Nk - 1) - base;
      const int lo = (W > 0 ? qrow + off - W + 1 : 0) - base;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kb * 32 + (r / 4) * 8 + (r % 4);
          if (kk > lim || (WINDOW && kk < lo)) sacc[kb][r] = -INFINITY;
        }
    };

    bool pending = false;  // wave-uniform: a rescale of O is due
    float pend_alpha = 1.f;

    // O^T += V(t)^T P(t) for the V tile in buffer vb (16 MFMAs).
    auto pv = [&](const bf16x8_t (&pp)[4], int vb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[vb] + v_off(kk, 0, db)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[vb] + v_off(kk, 1, db)));
          const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[kk], oacc[db], 0, 0, 0);
        }
    };

    // One pipeline stage t: softmax of tile t (scores in sc, weights out to pc)
    // on the vector ALUs, while the matrix cores run QK^T of tile t+1 (into sn)
    // and PV of tile t-1 (weights pp, V in buffer (t-1)&1).  The direct loads
    // of K(t+2) and V(t) fly during the whole stage.
    // The start of stage t: the direct loads of K(t+2) and V(t), then the
    // rescale decided in the previous stage, which applies to O once PV(t-2)
    // (its weights used the old reference) is in, i.e. now, before PV(t-1).
    auto stage_start = [&](int t) {
      if (t + 2 < te) copy_k(sm.k[t & 1], t + 2, eK);
      copy_v(sm.v[t & 1], t, eV);
      if (PAGED && one_block) {
        eK = entry(t + 3);
        eV = entry(t + 1);
        asm volatile("" ::: "memory");  // the lookups fly during this stage
      }
      if (pending) {
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= pend_alpha;
        pending = false;
      }
    };
    // Running max of tile t; a rescale it calls for applies to l now and to O
    // at the start of the next stage, after PV(t-1).  Returns the reference
    // the weights of tile t are taken against (also kept in mref).
    auto softmax_ref = [&](f32x16_t (&sc)[2], int t, float slack) {
      if (t >= n_clean || t < n_lo) mask(sc, t);
      float mx = sc[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = max_nan(mx, sc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = max_nan(mx, sc[1][r]);
      mx = halves_max_nan(mx) * c;
      // Rescale only when some row's max grows by more than `slack` (log2
      // units): (m, l, O) stays exact for any reference m within the slack
      // of the true max, and P is then at most 2^slack (fine in bf16).
      const float mn = max_nan(m, mx);
      if (__any(mn > m + slack)) {
        pend_alpha = fast_exp2(m - ((mn == -INFINITY) ? 0.f : mn));
        pending = true;
        l0 *= pend_alpha;
        l1 *= pend_alpha;
        m = mn;
      }
      mref = (m == -INFINITY) ? 0.f : m;
      return mref;
    };
    // S(t) again, from K in global memory: the same MFMAs on the same operands
    // as qk() on the LDS tile, so the same scores (rows outside [kbeg, Nk) are
    // read clamped, as the tile copies do, and masked afterwards).
    auto qk_global = [&](f32x16_t (&sacc)[2], int t) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int tok = min(max(t * kBN + kb * 32 + col, kbeg), Nk - 1);
        const uint16_t* kr;
        if constexpr (PAGED)
          kr = kg + ((size_t)trow[tok >> lbs] * bsz + (tok & (bsz - 1))) * slot_elems;
        else
          kr = kg + (size_t)tok * D;
        bf16x8_t kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8_t*>(kr + ks * 16 + hl * 8);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], ks == 0 ? f32x16_t{} : sacc[kb], 0, 0, 0);
        asm volatile("" ::: "memory");  // one key block's operands in registers at a time
      }
    };
    auto stage_end = [&]() {
      wait_all_vmem();  // this wave's direct loads have landed
      __syncthreads();  // ... and every other wave's
    };

    auto stage = [&](f32x16_t (&sc)[2], f32x16_t (&sn)[2], const bf16x8_t (&pp)[4], bf16x8_t (&pc)[4], int t,
                     bool with_pv) {
      const int kb_next = (t + 1) & 1;  // K(t+1)
      stage_start(t);

      // Operands of group j of the interleave below (QK^T k-step j % KS of
      // key block j / KS, and PV MFMA j), read from LDS one group ahead of
      // their MFMAs so that no MFMA waits for an LDS read it just issued.
      auto k_operand = [&](int j) {
        return *reinterpret_cast<const bf16x8_t*>(&sm.k[kb_next][k_off(j / KS, j % KS)]);
      };
      auto v_operand = [&](int j) {
        const int kk = j / DB, db = j % DB;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[(t - 1) & 1] + v_off(kk, 0, db)));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm.v[(t - 1) & 1] + v_off(kk, 1, db)));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t ka_n = k_operand(0), va_n{};
      if (with_pv) va_n = v_operand(0);

      // The weights of tile t are taken against the reference as it stands;
      // the tile's own max is looked at only if they come out too large
      // (below).  With a sliding window, whose rows find their first keys
      // tiles apart, the max comes first as before.
      float mu;
      if constexpr (WINDOW) {
        mu = softmax_ref(sc, t, kSlack);
      } else {
        if (t >= n_clean || t < n_lo) mask(sc, t);
        mu = mref;
      }

      // ---- matrix cores: S(t+1) and O += V(t-1) P(t-1); vector ALUs: P(t),
      // packed to bf16 pairs as they are made.  PV(t-1) has 4 * DB = 2 * KS
      // MFMAs, as many as QK^T: one per k-step.
      u32x4_t w[4];
      float ps0 = 0.f, ps1 = 0.f;  // this lane's sums of the tile's weights
#pragma unroll
      for (int j = 0; j < 2 * KS; ++j) {
        const int kb = j / KS, ks = j % KS;
        const bf16x8_t ka = ka_n, va = va_n;
        if (j + 1 < 2 * KS) {
          ka_n = k_operand(j + 1);
          if (with_pv) va_n = v_operand(j + 1);
        }
        sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], ks == 0 ? f32x16_t{} : sn[kb], 0, 0, 0);
        if (with_pv) oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[j / DB], oacc[j % DB], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < VPS; i += 2) {
          const int r = ks * VPS + i;  // register r of block kb: element r % 8 of half r / 8
          const float p0 = fast_exp2(fmaf(sc[kb][r], c, -mu));
          const float p1 = fast_exp2(fmaf(sc[kb][r + 1], c, -mu));
          if constexpr (WINDOW) {
            l0 += p0;
            l1 += p1;
          } else {
            ps0 += p0;
            ps1 += p1;
          }
          w[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16x2(p0, p1);
        }
        // interleave: each MFMA, then some of the next group's LDS reads (K
        // and the first V^T half after the first, the second V^T half after
        // the second), then half of the vector work
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);  // VALU incl. transcendental
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
      }
      // A lane's sum above 2^kSlack (as any weight above 2^kSlack makes it),
      // or a row still without a reference: the tile again, against its
      // exact max.  NaN sums (NaN scores) pass, as NaN maxima do.
      if (!WINDOW && __any(ps0 + ps1 > kSumMax || m == -INFINITY)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pin(w[i]);  // the first weights are made among the MFMAs all the same
        qk_global(sc, t);
        const float mu2 = softmax_ref(sc, t, 0.f);
        ps0 = ps1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(sc[kb][r], c, -mu2));
            const float p1 = fast_exp2(fmaf(sc[kb][r + 1], c, -mu2));
            ps0 += p0;
            ps1 += p1;
            w[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16x2(p0, p1);
          }
      }
      if constexpr (!WINDOW) {
        l0 += ps0;
        l1 += ps1;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pin(w[i]);
        pc[i] = __builtin_bit_cast(bf16x8_t, w[i]);
      }
      pin(l0);
      pin(l1);
      stage_end();
    };

    // The last stages of a wave near the causal diagonal.  Wave w's rows see
    // no key of tiles te_w and later (their weights would be exact zeros):
    // once S(te_w) would be next, the wave drops the products that only such
    // tiles feed and keeps copying its share of the tiles and meeting the
    // barriers.  SOFTMAX: the weights of tile t (sc -> pc); PV: O += V(t-1)
    // P(t-1) (pp), each V^T operand read one MFMA ahead.
    auto stage_part = [&](f32x16_t (&sc)[2], const bf16x8_t (&pp)[4], bf16x8_t (&pc)[4], int t, auto softmax,
                          auto with_pv) {
      stage_start(t);
      if constexpr (decltype(softmax)::value) {
        const float mu = softmax_ref(sc, t, kSlack);
        u32x4_t w[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(fmaf(sc[kb][r], c, -mu));
            const float p1 = fast_exp2(fmaf(sc[kb][r + 1], c, -mu));
            l0 += p0;
            l1 += p1;
            w[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16x2(p0, p1);
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) pc[i] = __builtin_bit_cast(bf16x8_t, w[i]);
      }
      if constexpr (decltype(with_pv)::value) {
        const uint16_t* vt = sm.v[(t - 1) & 1];
        auto v_op = [&](int j) {
          const int kk = j / DB, db = j % DB;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + v_off(kk, 0, db)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + v_off(kk, 1, db)));
          return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8_t va_n = v_op(0);
#pragma unroll
        for (int j = 0; j < 4 * DB; ++j) {
          const bf16x8_t va = va_n;
          if (j + 1 < 4 * DB) va_n = v_op(j + 1);
          oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[j / DB], oacc[j % DB], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      stage_end();
    };

    f32x16_t s_a[2], s_b[2];
    bf16x8_t p_a[4], p_b[4];

    // prologue: K(0) -> K buffer 0, K(1) -> K buffer 1.  The drain is
    // unconditional so that, on every path into the loop, the Q fragments are
    // known to have arrived (otherwise each QK^T MFMA waits on vmcnt).
    // Tiles are numbered from the start of the sequence; the workgroup visits
    // [tb, te) and buffer parity follows the tile number.
    if (te > tb) {
      const bool look = PAGED && one_block;
      copy_k(sm.k[tb & 1], tb, look ? entry(tb) : 0);
      if (te > tb + 1) copy_k(sm.k[(tb + 1) & 1], tb + 1, look ? entry(tb + 1) : 0);
      if (look) {
        eK = entry(tb + 2);
        eV = entry(tb);
      }
    }
    wait_all_vmem();
    __syncthreads();
    if (te > tb && tl == tb) qk(s_a, tb & 1);
    __syncthreads();  // K buffer of tile tb is refilled by the first stage

    if (te > tb) {
      using yes = std::true_type;
      using no = std::false_type;
      // a late window start: copies and barriers only, then S(tl) alone; the
      // register buffers then alternate from tl as they would from tb
      for (int u = tb; u < tl - 1; ++u) stage_part(s_b, p_a, p_b, u, no{}, no{});
      if (tl > tb) {
        stage_start(tl - 1);
        qk(s_a, tl & 1);
        stage_end();
      }
      // the wave's first tile: its exact max first, so that its weights pass
      // the check
      if constexpr (!WINDOW) softmax_ref(s_a, tl, 0.f);
      stage(s_a, s_b, p_b, p_a, tl, false);
      int t = tl + 1;
      // full stages while S(t+1) still has a key this wave sees
      const int t_full = min(te, te_w);
      for (; t + 1 < t_full; t += 2) {
        stage(s_b, s_a, p_a, p_b, t, true);
        stage(s_a, s_b, p_b, p_a, t + 1, true);
      }
      const int t_loop = t;  // stages from here on alternate buffers as stage t of the loop would
      if (t < te && t == te_w - 1) {  // weights of this wave's last tile and PV(t-1), then PV(t)
        stage_part(s_b, p_a, p_b, t, yes{}, yes{});
        if (++t < te) stage_part(s_a, p_b, p_a, t++, no{}, yes{});
      } else if (t < te && t == te_w) {  // PV of this wave's last tile
        stage_part(s_b, p_a, p_b, t++, no{}, yes{});
      }
      for (; t < te; ++t) stage_part(s_b, p_a, p_b, t, no{}, no{});  // copies and barriers only
      // drain: a due rescale, then PV of the last tile when this wave sees it
      if (pending) {
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= pend_alpha;
      }
      if (te_w >= te) {
        if (t_loop < te) pv(p_b, (te - 1) & 1);
        else pv(p_a, (te - 1) & 1);
      }
    }

    // ---- epilogue: one division, bf16 output, natural-log LSE.  O leaves
    // through LDS: each wave writes its 32 rows there as the accumulator holds
    // them (lane: one row, 8 bytes of a chunk) and reads them back whole-row
    // (lane: one 16-byte chunk), so that each global store covers 1 KiB of
    // consecutive rows instead of 16 bytes of 32 rows.  Chunk c of row r sits
    // at c ^ k_swz(r): the whole-chunk reads are conflict-free, and the 8-byte
    // writes cost the LDS about 64 conflict cycles per wave and tile (1.4% of
    // its active cycles, measured).
    const float lt = halves_sum(l0 + l1);
    const float inv = bad ? __builtin_nanf("") : lt > 0.f ? 1.f / lt : 0.f;
    __syncthreads();  // every wave's last PV has read its V tile
    // The lane's row and lane index pass through an empty statement, so that
    // the swizzled addresses below are formed here and not kept in registers
    // across the tile loop.
    int ecol = col, elane = lane;
    asm volatile("" : "+v"(ecol), "+v"(elane));
    uint16_t* ot = sm.o[wave];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2_t w;
        w[0] = pack_bf16x2(oacc[db][q4 * 4 + 0] * inv, oacc[db][q4 * 4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][q4 * 4 + 2] * inv, oacc[db][q4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(ot + ecol * D + (((db * 4 + q4) ^ k_swz<D>(ecol)) * 8) + hl * 4) = w;
      }
    // The output goes out with non-temporal stores: written through, it does
    // not sit dirty in L2 at the end of the launch (measured on MI355X: ~1%
    // shorter launches at N = 4096, where the last tile's output is written
    // right before the kernel ends).
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    uint16_t* obase = reinterpret_cast<uint16_t*>(a.o) + ((size_t)(b * a.Hq + hq) * a.Nq + q0 + pw) * D;
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int u = i * 64 + elane, r = u / CPR, ch = u % CPR;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ot + r * D + ((ch ^ k_swz<D>(r)) * 8));
      if (q0 + pw + r < a.Nq) __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(obase + r * D + ch * 8));
    }
    if (a.lse && hl == 0 && qrow < a.Nq)
      a.lse[(size_t)(b * a.Hq + hq) * a.Nq + qrow] = bad ? __builtin_nanf("") : lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  };
  if (single >= 0) {
    run_tile(single);
    return;
  }
  run_tile(nqb - 1 - pr);
  if (pr < nqb - 1 - pr) {
    __syncthreads();  // the first tile's last LDS reads are done
    run_tile(pr);
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int hw = heads_per_workgroup(a.Hq / a.Hkv);
  const int P = kBM / hw;  // query positions per tile
  const int nqb = (a.Nq + P - 1) / P;
  // several cached sequences (lengths known only to the device): single query
  // tiles, longest first; otherwise pairs of query tiles
  const int lpt = a.seq_lens != nullptr && a.B > 1;
  const long long grid = (long long)(lpt ? nqb : (nqb + 1) / 2) * (a.Hq / hw) * a.B;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool paged = a.block_table != nullptr, win = a.window > 0;
#define FA_LAUNCH(DD, PG, WN) \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, PG, WN>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, nqb, lpt)
  if (a.d == 64) {
    if (paged) { if (win) FA_LAUNCH(64, true, true); else FA_LAUNCH(64, true, false); }
    else { if (win) FA_LAUNCH(64, false, true); else FA_LAUNCH(64, false, false); }
  } else {
    if (paged) { if (win) FA_LAUNCH(128, true, true); else FA_LAUNCH(128, true, false); }
    else { if (win) FA_LAUNCH(128, false, true); else FA_LAUNCH(128, false, false); }
  }
#undef FA_LAUNCH
  return hipGetLastError();
}

}  // namespace fa
