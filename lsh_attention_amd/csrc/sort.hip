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
//             first output slot of every (bucket, tile) (bucket totals, an
//             exclusive scan over buckets, the counts of earlier tiles) and the
//             tile's own order (a scan of its counts, each wave's offset within
//             a bucket's run); then each wave ranks its sub-tile's tokens in
//             order: the lanes holding the same bucket are found with one ballot
//             per key bit (4 vector instructions per bit), their rank is the
//             count of those lanes below this one (mbcnt), and a per-wave 16-bit
//             LDS counter per bucket carries the running offset.  The unsort
//             index is written from the walk (coalesced); the sorted index too,
//             or, with 256 buckets or more, the tile's sorted order is staged in
//             LDS and written afterwards as whole bucket runs.
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

template <bool STAGE>
__global__ __launch_bounds__(1024) void sort_scatter_kernel(const int32_t* __restrict__ buckets,
                                                            const int* __restrict__ hist,
                                                            int32_t* __restrict__ sorted_idx,
                                                            int32_t* __restrict__ undo_idx, int L, int n_b,
                                                            int n_h, int n_tiles, int nbits, int n_items) {
  extern __shared__ int sh[];
  __shared__ int wtot[2][16];  // per-wave sums of the two bucket scans
  const int waves = blockDim.x >> 6;
  const int npair = (waves + 1) >> 1;
  const int tile_len = waves * kSortWaveTokens;
  // Dynamic LDS (sort_scatter_lds): cw[npair][n_b] holds waves 2p (low half) and
  // 2p+1 (high half) of each bucket's count, later its running offset within
  // the tile's run of the bucket; tpos[b] = the tile's first sorted position of
  // bucket b; goff[b] = global slot minus tile position for bucket b; stage[t] =
  // the tile's t-th token in sorted order, as an offset from t0 (< 8192).
  uint32_t* cw = (uint32_t*)sh;
  int* tpos = sh + npair * n_b;
  int* goff = tpos + n_b;
  uint16_t* stage = (uint16_t*)(goff + n_b);
  // The tiles of one problem share an XCD, so the sorted-index writes of one
  // problem meet in one L2.
  const unsigned item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= (unsigned)n_items) return;
  const int bhr = (int)item / n_tiles, tile = (int)item % n_tiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = tile * tile_len, t1 = min(L, t0 + tile_len);
  const int w0 = t0 + wave * kSortWaveTokens, w1 = min(t1, w0 + kSortWaveTokens);
  const int shift = 16 * (wave & 1);
  uint32_t* mycw = cw + (wave >> 1) * n_b;
  for (int b = threadIdx.x; b < npair * n_b; b += blockDim.x) cw[b] = 0u;
  __syncthreads();
  const int32_t* bk = buckets + (size_t)bhr * L;
  // 1. per-wave counts of its sub-tile (at most 512, so a 16-bit field); the
  //    buckets stay in registers for step 3
  constexpr int kPer = kSortWaveTokens / 64;
  int bv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = w0 + lane + 64 * k;
    bv[k] = i < w1 ? clamp_bucket(bk[i], n_b) : -1;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    if (bv[k] >= 0) atomicAdd(&mycw[bv[k]], 1u << shift);
  __syncthreads();
  // 2. Two exclusive scans over the buckets: of each bucket's total in the
  //    problem-round (its first output slot, plus its counts in earlier tiles)
  //    and of its count in this tile (its first position in the tile's sorted
  //    order); then each wave's offset within the tile's run of the bucket.
  //    Thread t owns the contiguous buckets [t*per, (t+1)*per).
  const int* hp = hist + (size_t)bhr * n_tiles * n_b;  // [tile][bucket] counts
  const int nthr = (int)blockDim.x;
  const int per = (n_b + nthr - 1) / nthr;
  const int bb0 = min(n_b, (int)threadIdx.x * per), bb1 = min(n_b, bb0 + per);
  int gmine = 0, tmine = 0;
  for (int b = bb0; b < bb1; ++b) {
    for (int t = 0; t < n_tiles; ++t) gmine += hp[(size_t)t * n_b + b];
    for (int q = 0; q < npair; ++q) {
      const uint32_t w = cw[q * n_b + b];
      tmine += (int)(w & 0xFFFFu) + (int)(w >> 16);
    }
  }
  int gin = gmine, tin = tmine;
  for (int off = 1; off < 64; off <<= 1) {
    const int yg = __shfl_up(gin, off), yt = __shfl_up(tin, off);
    if (lane >= off) {
      gin += yg;
      tin += yt;
    }
  }
  if (lane == 63) {
    wtot[0][wave] = gin;
    wtot[1][wave] = tin;
  }
  __syncthreads();
  int grun = gin - gmine, trun = tin - tmine;
  for (int w = 0; w < wave; ++w) {
    grun += wtot[0][w];
    trun += wtot[1][w];
  }
  const int r = bhr % n_h, bh = bhr / n_h;
  for (int b = bb0; b < bb1; ++b) {
    int before = 0, total = 0;
    for (int t = 0; t < n_tiles; ++t) {
      const int c = hp[(size_t)t * n_b + b];
      before += t < tile ? c : 0;
      total += c;
    }
    tpos[b] = trun;
    goff[b] = r * L + grun + before - trun;
    int o = 0;  // waves' offsets within the tile's run of bucket b, in wave order
    for (int q = 0; q < npair; ++q) {
      const uint32_t w = cw[q * n_b + b];
      const int lo = (int)(w & 0xFFFFu), hi = (int)(w >> 16);
      cw[q * n_b + b] = (uint32_t)o | ((uint32_t)(o + lo) << 16);
      o += lo + hi;
    }
    grun += total;
    trun += o;
  }
  __syncthreads();
  // 3. Ordered walk, 64 tokens at a time: each token's position in the tile's
  //    sorted order and its global slot; the unsort index is written here
  //    (coalesced), the sorted index either here too (STAGE false) or, staged
  //    in LDS, after the walk.
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
    // this wave's running offset in the bucket's run (its own half of the word;
    // the other wave of the pair only adds to the other half, without carry)
    const int first = act ? (int)((mycw[b] >> shift) & 0xFFFFu) : 0;
    if (act && rank == 0) atomicAdd(&mycw[b], (uint32_t)(__popc(mlo) + __popc(mhi)) << shift);
    if (act) {
      const int t = tpos[b] + first + rank;
      const int g = goff[b] + t;
      uidx[i] = g;
      if constexpr (STAGE)
        stage[t] = (uint16_t)(i - t0);
      else
        sidx[g] = i;
    }
  }
  if constexpr (!STAGE) return;
  __syncthreads();
  // 4. The sorted index of the tile, written in sorted order: consecutive threads
  //    write consecutive slots within each bucket's run (the token's bucket is
  //    read again from the bucket array, which this block just read).
  const int cnt = t1 - t0;
  for (int t = (int)threadIdx.x; t < cnt; t += (int)blockDim.x) {
    const int i = t0 + (int)stage[t];
    sidx[goff[clamp_bucket(bk[i], n_b)] + t] = i;
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
  // With 256 buckets or more, the lanes of a 64-token step hold different
  // buckets, so writing the sorted index from the walk touches a line per lane;
  // staging the tile's order and writing whole bucket runs then pays
  // (long_seq_64k 33.5 -> 30.6 us, peaked_vmf_16k 29.2 -> 23.6 us).  With fewer
  // buckets the walk's writes already share lines and the extra phase costs more
  // (causal_lm_4k 11.7 -> 13.3 us).
  if (n_b >= 256)
    sort_scatter_kernel<true><<<xcd_grid(nt * BHR), 64 * waves, sort_scatter_lds(waves, n_b), s>>>(
        buckets, hist, sorted_idx, undo_idx, L, n_b, n_h, nt, nbits, nt * BHR);
  else
    sort_scatter_kernel<false><<<xcd_grid(nt * BHR), 64 * waves, sort_scatter_lds(waves, n_b), s>>>(
        buckets, hist, sorted_idx, undo_idx, L, n_b, n_h, nt, nbits, nt * BHR);
  return hipGetLastError();
}

}  // namespace lsh
