// Internal declarations shared by the gfx950 kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lsh_attn.h"

namespace lsh {

constexpr int kD = 64;          // head dimension handled by the kernels
constexpr int kChunk = 64;      // chunk length handled by the attention kernel
constexpr int kMaxHashes = 16;  // upper bound on hash rounds
constexpr int kMaxBuckets = 4096;
constexpr int kSortWaveTokens = 512;  // tokens ranked by one wave of the sort scatter
constexpr int kMaxLen = 1 << 24; // rows are addressed with 32-bit byte offsets

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Attention logits are handled in base 2: logit * log2(e) = (x_i . x_j) * ks_j with
// ks_j = log2(e) / (8 |x_j|) (scale 1/sqrt(64), key norm floored at 1e-12), and every
// logit of query i is at most M_i = log2(e) |x_i| / 8.  From |x|^2: (ks, M).
constexpr float kScale2 = 0.125f * 1.4426950408889634f;
__device__ inline float2 token_scale(float norm2) {
  const float nrm = __builtin_amdgcn_sqrtf(norm2);
  return make_float2(kScale2 * __builtin_amdgcn_rcpf(fmaxf(nrm, 1e-12f)), kScale2 * nrm);
}

// Work-item order for launches whose consecutive items share data.  The chip's 8
// XCDs each have their own L2, and workgroups are handed to XCDs round-robin by
// block index.  A launch of xcd_grid(n) blocks that maps block b to item
// xcd_item(b, gridDim.x) (items >= n return at once) runs items
// [x*g/8, (x+1)*g/8) on XCD x, in order (g = xcd_grid(n)).
constexpr unsigned kXcds = 8;
inline unsigned xcd_grid(unsigned n) { return (n + kXcds - 1) / kXcds * kXcds; }
__device__ inline unsigned xcd_item(unsigned b, unsigned grid) { return (b % kXcds) * (grid / kXcds) + b / kXcds; }

// Columns of the transposed rotation, padded to whole 64-column staging blocks
// (two 32-column MFMA tiles).
inline int padded_half(int n_b) { return n_b == 1 ? 0 : (int)align_up((size_t)(n_b / 2), 64); }
// LDS of one sort-scatter block of w waves: per-wave 16-bit bucket counters
// (two waves per word), two ints per bucket (the tile's first sorted position of
// the bucket and its offset to the global slot), and the tile's staged order
// (16-bit token offsets).
inline size_t sort_scatter_lds(int w, int n_b) {
  return (size_t)((w + 1) / 2) * n_b * 4 + (size_t)n_b * 8 + (size_t)w * kSortWaveTokens * 2;
}
// Waves per sort tile: as many as the sequence needs, at most 16, and no more
// than fit the scatter block's LDS in 63.5 KiB.  Larger tiles give longer runs
// of consecutive output slots per bucket (fewer partial-line writes).
inline int sort_waves(int L, int n_b) {
  const int need = (L + kSortWaveTokens - 1) / kSortWaveTokens;
  int w = need < 16 ? (need < 1 ? 1 : need) : 16;
  while (w > 1 && sort_scatter_lds(w, n_b) > 65024) --w;
  return w;
}
inline int sort_tile(int L, int n_b) { return kSortWaveTokens * sort_waves(L, n_b); }
inline int sort_tiles(int L, int n_b) { return (L + sort_tile(L, n_b) - 1) / sort_tile(L, n_b); }

// ---- launchers (stream-ordered, no synchronisation) ----
// Rotation transpose [n_h][D][half] -> [n_h][halfp][D] with zero padding, the
// largest column norm per 64-column block (colmax: n_h * ceil(halfp/64)
// floats), and the reset of the uncertified-token count.
inline int colmax_blocks(int n_b) { return (padded_half(n_b) + 63) / 64; }
hipError_t launch_prep(const void* rot, void* rot_t, float* colmax, int* fix_count, int n_h, int n_b,
                       lsh_dtype dt, hipStream_t s);
// token_scales (nullable): per token (key scale, query bound) for the attention pass.
hipError_t launch_hash(const void* qk, const void* rot_t, const float* colmax, int32_t* buckets,
                       int* fix_queue, int* fix_count, float2* token_scales, int BH, int L, int n_b,
                       int n_h, lsh_dtype dt, hipStream_t s);
hipError_t launch_fixup(const void* qk, const void* rot_t, const float* colmax, int32_t* buckets,
                        const int* fix_queue, const int* fix_count, int L, int n_b, int n_h, lsh_dtype dt,
                        hipStream_t s);
hipError_t launch_fill_zero(int32_t* p, size_t n, hipStream_t s);

hipError_t launch_sort_hist(const int32_t* buckets, int* hist, int BHR, int L, int n_b,
                            hipStream_t s);
hipError_t launch_sort_scatter(const int32_t* buckets, const int* hist, int32_t* sorted_idx,
                               int32_t* undo_idx, int BHR, int L, int n_b, int n_h,
                               hipStream_t s);

// The per-slot attention rows are written once and read once, by the combine.
// When they outgrow the chip's 256 MiB last-level cache they are written and
// read with non-temporal accesses, which keeps them from evicting the QK and V
// rows that the attention gathers again in every round.
inline bool stream_slot_rows(int BH, int L, int n_h, lsh_dtype dt) {
  return (size_t)BH * n_h * L * kD * (dt == LSH_BF16 ? 2 : 4) >= (256ull << 20);
}

// Outputs per sorted slot ([BH][n_h*L][64], [BH][n_h*L]).  token_scales (nullable): per
// token (key scale, query bound) from the hash pass.  attend: 0, or the
// LSH_ATTEND_* bits; buckets ([BH][n_h][L]) are read with LSH_ATTEND_SAME_BUCKET,
// undo_idx ([BH][n_h][L]) with LSH_ATTEND_DEDUP, which first writes a token-major
// record to tok_rec (BH * L * n_h ints of scratch); nullptr where unused.
hipError_t launch_chunk_attn(const void* qk, const void* v, const int32_t* sorted_idx,
                             void* o_out, float* lse_out, const float2* token_scales,
                             const int32_t* buckets, const int32_t* undo_idx, int32_t* tok_rec,
                             int BH, int L, int n_h, int causal, int attend, lsh_dtype dt,
                             hipStream_t s);

// Unsort + combine from the per-slot layout, through undo_idx.
hipError_t launch_combine(const void* o_sorted, const float* lse_sorted, const int32_t* undo_idx,
                          void* out, float* lse_out, int BH, int L, int n_h, lsh_dtype dt,
                          hipStream_t s);

}  // namespace lsh
