// Steps 4-5 of the shared-QK LSH attention forward pass: unsort the per-round
// results and combine the rounds.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer): several hash rounds
// with independent rotations are unioned to raise recall.  The union is taken
// as one softmax over all rounds' windows, which, given each round's output
// o_r(i) and log-sum-exp lse_r(i), is
//   LSE_i = logsumexp_r lse_r(i),  out_i = sum_r exp(lse_r(i) - LSE_i) o_r(i).
//
// gfx950 design: a pure gather-and-reduce, HBM-bound.  Each token is handled
// by a group of lanes that each own 16 bytes of the 64-wide row (8 lanes for
// bf16 rows, 16 for fp32), so every round's row is one fully used 128- or
// 256-byte read; all rounds' loads are issued before any is used.
#include "lsh_internal.h"

namespace lsh {

namespace {

template <bool BF16, int NH>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o_sorted_v,
                                                      const float* __restrict__ lse_sorted,
                                                      const int32_t* __restrict__ undo_idx,
                                                      void* __restrict__ out_v, float* __restrict__ lse_out,
                                                      int L, int n_h_rt, size_t n_tokens, bool nt_in,
                                                      bool xcd_order) {
  constexpr int kLanesPerTok = BF16 ? 8 : 16;
  constexpr int kMaxH = NH > 0 ? NH : kMaxHashes;
  const int n_h = NH > 0 ? NH : n_h_rt;
  const size_t blk = xcd_order ? xcd_item(blockIdx.x, gridDim.x) : blockIdx.x;
  const size_t gid = blk * blockDim.x + threadIdx.x;
  const size_t tok = gid / kLanesPerTok;
  const int sub = (int)(gid % kLanesPerTok);
  if (tok >= n_tokens) return;
  const size_t bh = tok / L;
  const int i = (int)(tok % L);
  const size_t n_slots = (size_t)n_h * L;
  const int32_t* u = undo_idx + bh * n_slots + i;

  int g[kMaxH];
  float l[kMaxH];
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) g[r] = (int)min((uint32_t)u[(size_t)r * L], (uint32_t)(n_slots - 1));  // in-bounds guard
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) l[r] = lse_sorted[bh * n_slots + g[r]];
  uint4 raw[kMaxH];
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) {
      const char* row = (const char*)o_sorted_v + ((bh * n_slots + g[r]) * kD) * (BF16 ? 2 : 4);
      if (nt_in) {
        const u32x4 t = __builtin_nontemporal_load((const u32x4*)(row + 16 * sub));
        raw[r] = make_uint4(t[0], t[1], t[2], t[3]);
      } else {
        raw[r] = *(const uint4*)(row + 16 * sub);
      }
    }
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) m = fmaxf(m, l[r]);
  float w[kMaxH];
  float tot = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) {
      w[r] = __expf(l[r] - m);
      tot += w[r];
    }
  const float inv = __builtin_amdgcn_rcpf(tot);
  constexpr int kE = BF16 ? 8 : 4;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxH; ++r)
    if (r < n_h) {
      const float wr = w[r] * inv;
      const uint32_t ww[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
      if constexpr (BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = fmaf(wr, __uint_as_float(ww[k] << 16), acc[2 * k]);
          acc[2 * k + 1] = fmaf(wr, __uint_as_float(ww[k] & 0xFFFF0000u), acc[2 * k + 1]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = fmaf(wr, __uint_as_float(ww[k]), acc[k]);
      }
    }
  char* orow = (char*)out_v + (tok * kD) * (BF16 ? 2 : 4);
  if constexpr (BF16) {
    uint32_t pk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      pk[k] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * k]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * k + 1]) << 16);
    *(uint4*)(orow + 16 * sub) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  } else {
    *(float4*)(orow + 16 * sub) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  if (lse_out != nullptr && sub == 0) lse_out[tok] = m + __logf(tot);
}

template <bool BF16>
hipError_t launch_combine_t(const void* o_sorted, const float* lse_sorted, const int32_t* undo_idx, void* out,
                            float* lse_out, int BH, int L, int n_h, hipStream_t s) {
  const size_t n_tokens = (size_t)BH * L;
  const size_t threads = n_tokens * (BF16 ? 8 : 16);
  const bool nt = stream_slot_rows(BH, L, n_h, BF16 ? LSH_BF16 : LSH_F32);  // as the attention wrote them
  // Rows that stay in the last-level cache between the two kernels: each XCD
  // takes a contiguous range of tokens (causal_lm_4k 31.8 -> 27.1 us); streamed
  // rows keep the plain order.
  const bool xo = !nt;
  const unsigned n_blk = (unsigned)((threads + 255) / 256);
  const unsigned grid = xo ? xcd_grid(n_blk) : n_blk;
#define LSH_COMBINE_CASE(NHV)                                                                              \
  case NHV:                                                                                                \
    combine_kernel<BF16, NHV><<<grid, 256, 0, s>>>(o_sorted, lse_sorted, undo_idx, out, lse_out, L, n_h,   \
                                                   n_tokens, nt, xo);                                          \
    break;
  switch (n_h) {
    LSH_COMBINE_CASE(1)
    LSH_COMBINE_CASE(2)
    LSH_COMBINE_CASE(3)
    LSH_COMBINE_CASE(4)
    LSH_COMBINE_CASE(8)
    default:
      combine_kernel<BF16, 0><<<grid, 256, 0, s>>>(o_sorted, lse_sorted, undo_idx, out, lse_out, L, n_h,
                                                   n_tokens, nt, xo);
  }
#undef LSH_COMBINE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const void* o_sorted, const float* lse_sorted, const int32_t* undo_idx, void* out,
                          float* lse_out, int BH, int L, int n_h, lsh_dtype dt, hipStream_t s) {
  if (dt == LSH_BF16) return launch_combine_t<true>(o_sorted, lse_sorted, undo_idx, out, lse_out, BH, L, n_h, s);
  return launch_combine_t<false>(o_sorted, lse_sorted, undo_idx, out, lse_out, BH, L, n_h, s);
}

}  // namespace lsh
