// Step 2 of the shared-QK LSH attention forward pass: sort tokens by bucket.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer): tokens are sorted by
// bucket so bucket-mates become contiguous.  The key here is (round, bucket,
// position): a stable sort of each round's positions by bucket.  Since the key
// is unique the permutation is fully determined.
//
// With at most 4096 buckets this is a counting sort, O(n) rather than the
// explainer's O(n log n) comparison sort, in two launches per call:
//   hist    - per (problem, round, tile of sort_tile() tokens) bucket histogram
//             in LDS, stored hist[bhr][tile][bucket] (coalesced rows);
//   scatter - each block first turns its problem's tile histograms into the
//             first output slot of every (bucket, tile, wave) (bucket totals,
//             an exclusive scan over buckets, the counts of earlier tiles and
//             waves); then each wave ranks its sub-tile's tokens in order: the
//             lanes holding the same bucket are found with one ballot per key
//             bit (4 vector instructions per bit), their rank is the count of
//             those lanes below this one (mbcnt), and a per-wave LDS counter per
//             bucket carries the running offset.
// Bucket values outside [0, n_b) are clamped to n_b - 1 (callers must not
// pass them; clamping only keeps every write in bounds).
#include "lsh_internal.h"

namespace lsh {

namespace {

__device__ inline int clamp_bucket(int32_t b, int n_b) { return (int)min((uint32_t)b, (uint32_t)(n_b - 1)); }

__global__ __launch_bounds__(1024) void sort_hist_kernel(const int32_t* __restrict__ buckets,
                                                        int* __restrict__ hist, int L, int n_b,
                                                        int n_tiles, int tile_len, int n_items) {
  extern __shared__ int sh[];  // n_b counters
  const unsigned item = xcd_item(blockIdx.x, gridDim.x);  // the tiles of one problem share an XCD
  if (item >= (unsigned)n_items) return;
  const int bhr = (int)item / n_tiles, tile = (int)item % n_tiles;
  for (int b = threadIdx.x; b < n_b; b += blockDim.x) sh[b] = 0;
  __syncthreads();
  const int t0 = tile * tile_len, t1 = min(L, t0 + tile_len);
  const int32_t* bk = buckets + (size_t)bhr * L;
  for (int i = t0 + (int)threadIdx.x; i < t1; i += blockDim.x) atomicAdd(&sh[clamp_bucket(bk[i], n_b)], 1);
  __syncthreads();
  int* out = hist + ((size_t)bhr * n_tiles + tile) * n_b;
  for (int b = threadIdx.x; b < n_b; b += blockDim.x) out[b] = sh[b];
}

__global__ __launch_bounds__(1024) void sort_scatter_kernel(const int32_t* __restrict__ buckets,
                                                            const int* __restrict__ hist,
                                                            int32_t* __restrict__ sorted_idx,
                                                            int32_t* __restrict__ undo_idx, int L, int n_b,
                                                            int n_h, int n_tiles, int nbits, int n_items) {
  extern __shared__ int sh[];  // waves x n_b running offsets
  __shared__ int wtot[16];      // per-wave sums of the bucket scan
  const int waves = blockDim.x >> 6;
  // The tiles of one problem share an XCD, so the scattered writes of one
  // problem's sorted index meet in one L2 and leave it as whole lines.
  const unsigned item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= (unsigned)n_items) return;
  const int bhr = (int)item / n_tiles, tile = (int)item % n_tiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = tile * waves * kSortWaveTokens, t1 = min(L, t0 + waves * kSortWaveTokens);
  const int w0 = t0 + wave * kSortWaveTokens, w1 = min(t1, w0 + kSortWaveTokens);
  int* cnt = sh + wave * n_b;
  for (int b = threadIdx.x; b < waves * n_b; b += blockDim.x) sh[b] = 0;
  __syncthreads();
  const int32_t* bk = buckets + (size_t)bhr * L;
  // 1. per-wave counts of its sub-tile; the buckets stay in registers for step 3
  constexpr int kPer = kSortWaveTokens / 64;
  int bv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = w0 + lane + 64 * k;
    bv[k] = i < w1 ? clamp_bucket(bk[i], n_b) : -1;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (bv[k] >= 0) atomicAdd(&cnt[bv[k]], 1);
  __syncthreads();
  // 2. first slot of (bucket, wave) in the round's output: the totals of all
  //    smaller buckets, plus this bucket's counts in earlier tiles, plus its
  //    counts in the earlier waves of this tile.  Each block scans the problem's
  //    tile histograms itself (the same scan in every tile of the problem).
  //    Thread t owns the contiguous buckets [t*per, (t+1)*per).
  const int* hp = hist + (size_t)bhr * n_tiles * n_b;  // [tile][bucket] counts
  const int nthr = (int)blockDim.x;
  const int per = (n_b + nthr - 1) / nthr;
  const int bb0 = min(n_b, (int)threadIdx.x * per), bb1 = min(n_b, bb0 + per);
  int mine = 0, before1 = 0;  // per == 1: the one bucket's total and its count in earlier tiles
  if (per == 1) {
    if (bb0 < bb1)
      for (int t = 0; t < n_tiles; ++t) {
        const int c = hp[(size_t)t * n_b + bb0];
        before1 += t < tile ? c : 0;
        mine += c;
      }
  } else {
    for (int b = bb0; b < bb1; ++b)
      for (int t = 0; t < n_tiles; ++t) mine += hp[(size_t)t * n_b + b];
  }
  // exclusive scan of `mine` over the threads of the block
  int incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int w = 0; w < wave; ++w) run += wtot[w];
  for (int b = bb0; b < bb1; ++b) {
    int before = before1, total = mine;
    if (per != 1) {
      before = total = 0;
      for (int t = 0; t < n_tiles; ++t) {
        const int c = hp[(size_t)t * n_b + b];
        before += t < tile ? c : 0;
        total += c;
      }
    }
    int slot = run + before;
    for (int w = 0; w < waves; ++w) {
      const int c = sh[w * n_b + b];
      sh[w * n_b + b] = slot;
      slot += c;
    }
    run += total;
  }
  __syncthreads();
  // 3. ordered walk, 64 tokens at a time.
  const int r = bhr % n_h, bh = bhr / n_h;
  int32_t* sidx = sorted_idx + (size_t)bh * n_h * L;
  int32_t* uidx = undo_idx + (size_t)bhr * L;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = w0 + 64 * k + lane;
    const bool act = bv[k] >= 0;  // i < w1
    const int b = act ? bv[k] : 0;
    // Lanes holding the same bucket: the active lanes whose ballot of every key
    // bit agrees with this lane's bit.  s = bit t of b as 0 or all ones, so each
    // half of the mask takes one three-input bitwise instruction per bit.
    const uint64_t am = __ballot(act);
    uint32_t mlo = (uint32_t)am, mhi = (uint32_t)(am >> 32);
    for (int t = 0; t < nbits; ++t) {
      const uint32_t s = (uint32_t)__builtin_amdgcn_sbfe(b, (uint32_t)t, 1u);
      const uint64_t bal = __ballot(s != 0u);
      mlo &= ~((uint32_t)bal ^ s);
      mhi &= ~((uint32_t)(bal >> 32) ^ s);
    }
    const int rank = (int)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));  // same-bucket lanes below
    const int first = act ? cnt[b] : 0;
    if (act && rank == 0) cnt[b] = first + __popc(mlo) + __popc(mhi);
    if (act) {
      const int g = r * L + first + rank;
      sidx[g] = i;
      uidx[i] = g;
    }
  }
}

}  // namespace

hipError_t launch_sort_hist(const int32_t* buckets, int* hist, int BHR, int L, int n_b, hipStream_t s) {
  const int nt = sort_tiles(L, n_b);
  const int threads = min(1024, sort_tile(L, n_b));
  sort_hist_kernel<<<xcd_grid(nt * BHR), threads, n_b * sizeof(int), s>>>(buckets, hist, L, n_b, nt,
                                                                           sort_tile(L, n_b), nt * BHR);
  return hipGetLastError();
}

hipError_t launch_sort_scatter(const int32_t* buckets, const int* hist, int32_t* sorted_idx,
                               int32_t* undo_idx, int BHR, int L, int n_b, int n_h, hipStream_t s) {
  const int nt = sort_tiles(L, n_b), waves = sort_waves(L, n_b);
  int nbits = 0;
  while ((1 << nbits) < n_b) ++nbits;
  sort_scatter_kernel<<<xcd_grid(nt * BHR), 64 * waves, waves * n_b * sizeof(int), s>>>(
      buckets, hist, sorted_idx, undo_idx, L, n_b, n_h, nt, nbits, nt * BHR);
  return hipGetLastError();
}

}  // namespace lsh
