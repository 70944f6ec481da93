// Step 3 of the shared-QK LSH attention forward pass: attention inside equal
// chunks of the sorted order.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer): after sorting, tokens
// are processed in equal chunks so each attends to its bucket-mates; queries
// and keys are the same vectors (shared-QK).  Here the sorted slots of all
// rounds form one round-major sequence of n_h*L slots, cut into chunks of 64;
// chunk c attends to chunk c-1 (cyclically over that sequence) and to itself.
// For query i and key j: logit = (x_i . x_j / max(|x_j|, 1e-12)) / sqrt(64),
// j == i gets -1e5 (a token sees itself only when nothing else is left), and
// with the causal flag keys after the query's original position are dropped.
// Per slot the kernel writes the softmax-weighted sum of V and the logits'
// log-sum-exp.
//
// gfx950 design (one block of 4 waves walks a run of consecutive chunks of one
// (batch, head)):
//  * The 64 rows of x and v of each chunk are gathered once (128-byte rows,
//    addressed through sorted_idx) into LDS; the previous chunk's rows stay
//    resident from the previous iteration (two-slot ring), so each chunk is
//    read from HBM/L2 once per block instead of twice.
//  * S^T = K Q^T on MFMA (keys are MFMA rows, queries MFMA columns), so each
//    lane holds one query's logits for 4 consecutive keys per 16-key tile; the
//    softmax reductions are two cross-lane steps.
//  * O^T = V^T P^T on MFMA: the P^T operand is exactly the lane's own logits
//    (the K index is permuted to match), V is kept transposed in LDS.
//  * Key norms are applied to the fp32 logits (raw bf16 keys feed the MFMA),
//    so no rounded normalised keys enter the product.
//  * The softmax runs in base 2 on v_exp_f32.
#include "lsh_internal.h"

namespace lsh {

namespace {

constexpr int kChunksPerBlock = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <bool BF16>
struct AttnTraits;
template <>
struct AttnTraits<true> {
  using T = uint16_t;
  static constexpr int kXRow = 72;   // x rows in LDS: 64 dims + 8 pad (144 B)
  static constexpr int kVRow = 136;  // V^T rows in LDS: 128 keys + 8 pad (272 B)
  static constexpr int kPer16 = 8;   // elements per 16-byte load
};
template <>
struct AttnTraits<false> {
  using T = float;
  static constexpr int kXRow = 68;
  static constexpr int kVRow = 132;
  static constexpr int kPer16 = 4;
};

__device__ inline uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256) void chunk_attn_kernel(const typename AttnTraits<BF16>::T* __restrict__ qk,
                                                         const typename AttnTraits<BF16>::T* __restrict__ v,
                                                         const int32_t* __restrict__ sorted_idx,
                                                         typename AttnTraits<BF16>::T* __restrict__ o_sorted,
                                                         float* __restrict__ lse_sorted, int L, int n_slots,
                                                         int n_chunks, int blocks_per_bh) {
  using T = typename AttnTraits<BF16>::T;
  constexpr int kXRow = AttnTraits<BF16>::kXRow;
  constexpr int kVRow = AttnTraits<BF16>::kVRow;
  constexpr int kPer16 = AttnTraits<BF16>::kPer16;
  __shared__ __attribute__((aligned(16))) T sX[2][64 * kXRow];
  __shared__ __attribute__((aligned(16))) T sVT[64 * kVRow];  // [dim][64 * slot + key]
  __shared__ __attribute__((aligned(16))) float sInv[2][64];
  __shared__ __attribute__((aligned(16))) int sPos[2][64];

  const int bh = blockIdx.x / blocks_per_bh;
  const int c0 = (blockIdx.x % blocks_per_bh) * kChunksPerBlock;
  const int c1 = min(n_chunks, c0 + kChunksPerBlock);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15;  // query (column) of the MFMA tiles
  const int grp = lane >> 4;  // 4-key group within a 16-key tile

  const T* xq = qk + (size_t)bh * L * kD;
  const T* vq = v + (size_t)bh * L * kD;
  const int32_t* sidx = sorted_idx + (size_t)bh * n_slots;

  // Gather chunk c into ring slot `slot`: thread t loads 16 dims of row t/4.
  auto load_chunk = [&](int c, int slot) {
    const int row = threadIdx.x >> 2, quarter = threadIdx.x & 3;
    // Positions come from a permutation of [0, L); the clamp only keeps a
    // malformed index array from reading out of bounds.
    const int pos = (int)min((uint32_t)sidx[(size_t)c * kChunk + row], (uint32_t)(L - 1));
    const T* xr = xq + (size_t)pos * kD + 16 * quarter;
    const T* vr = vq + (size_t)pos * kD + 16 * quarter;
    float ss = 0.f;
    constexpr int kLoads = 16 / kPer16;
    uint4 xv[kLoads], vv[kLoads];
    for (int k = 0; k < kLoads; ++k) {
      xv[k] = *(const uint4*)(xr + k * kPer16);
      vv[k] = *(const uint4*)(vr + k * kPer16);
    }
    for (int k = 0; k < kLoads; ++k) {
      *(uint4*)(&sX[slot][row * kXRow + 16 * quarter + k * kPer16]) = xv[k];
      const uint32_t xw[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
      const uint32_t vw[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
      if constexpr (BF16) {
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(xw[e] << 16), hi = __uint_as_float(xw[e] & 0xFFFF0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
          const int d = 16 * quarter + k * 8 + 2 * e;
          sVT[d * kVRow + 64 * slot + row] = (uint16_t)(vw[e] & 0xFFFFu);
          sVT[(d + 1) * kVRow + 64 * slot + row] = (uint16_t)(vw[e] >> 16);
        }
      } else {
        for (int e = 0; e < 4; ++e) {
          const float f = __uint_as_float(xw[e]);
          ss = fmaf(f, f, ss);
          const int d = 16 * quarter + k * 4 + e;
          sVT[d * kVRow + 64 * slot + row] = __uint_as_float(vw[e]);
        }
      }
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (quarter == 0) {
      sInv[slot][row] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
      sPos[slot][row] = pos;
    }
  };

  load_chunk((c0 - 1 + n_chunks) % n_chunks, (c0 + 1) & 1);

  for (int c = c0; c < c1; ++c) {
    const int cur = c & 1, prv = cur ^ 1;
    load_chunk(c, cur);
    __syncthreads();

    const int qrow = 16 * wave + col;  // this lane's query row in the current chunk
    const int qpos = sPos[cur][qrow];

    // ---- S^T = K Q^T : 8 key tiles of 16 (tiles 0-3 previous chunk, 4-7 current) ----
    f32x4 acc[8];
    if constexpr (BF16) {
      const bf16x8 bq0 = *(const bf16x8*)(&sX[cur][qrow * kXRow + 8 * grp]);
      const bf16x8 bq1 = *(const bf16x8*)(&sX[cur][qrow * kXRow + 32 + 8 * grp]);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const T* kr = &sX[kt < 4 ? prv : cur][(16 * (kt & 3) + col) * kXRow];
        const bf16x8 a0 = *(const bf16x8*)(kr + 8 * grp);
        const bf16x8 a1 = *(const bf16x8*)(kr + 32 + 8 * grp);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bq0, z, 0, 0, 0);
        acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bq1, z, 0, 0, 0);
      }
    } else {
      // k-step s of 4 dims: lane group g feeds dim 16g + s.
      float bq[16];
      for (int s4 = 0; s4 < 4; ++s4) {
        const float4 t = *(const float4*)(&sX[cur][qrow * kXRow + 16 * grp + 4 * s4]);
        bq[4 * s4] = t.x; bq[4 * s4 + 1] = t.y; bq[4 * s4 + 2] = t.z; bq[4 * s4 + 3] = t.w;
      }
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const T* kr = &sX[kt < 4 ? prv : cur][(16 * (kt & 3) + col) * kXRow + 16 * grp];
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int s4 = 0; s4 < 4; ++s4) {
          const float4 t = *(const float4*)(kr + 4 * s4);
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(t.x, bq[4 * s4 + 0], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(t.y, bq[4 * s4 + 1], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(t.z, bq[4 * s4 + 2], z, 0, 0, 0);
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(t.w, bq[4 * s4 + 3], z, 0, 0, 0);
        }
        acc[kt] = z;
      }
    }

    // ---- logits in base 2, masks, row max ----
    constexpr float kScale = 0.125f * kLog2e;         // 1/sqrt(64), base 2
    constexpr float kSelf = -1.0e5f * kLog2e;          // self logit, base 2
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const int slot = kt < 4 ? prv : cur;
      const int kr0 = 16 * (kt & 3) + 4 * grp;
      const float4 inv = *(const float4*)(&sInv[slot][kr0]);
      const int4 kp = *(const int4*)(&sPos[slot][kr0]);
      const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
      const int kpos[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = acc[kt][e] * (iv[e] * kScale);
        if (kpos[e] == qpos) s = kSelf;
        if (CAUSAL && kpos[e] > qpos) s = -INFINITY;
        acc[kt][e] = s;
        mx = fmaxf(mx, s);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = __builtin_amdgcn_exp2f(acc[kt][e] - mx);
        acc[kt][e] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);

    // ---- O^T = V^T P^T ----
    f32x4 oacc[4];
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // K index (grp, e): e < 4 -> key 4 grp + e of tile 2ks; e >= 4 -> of tile 2ks + 1.
        bf16x8 bp;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bp[e] = (__bf16)acc[2 * ks][e];
          bp[4 + e] = (__bf16)acc[2 * ks + 1][e];
        }
        const int slot = ks < 2 ? prv : cur;
        const int kc0 = 64 * slot + 16 * ((2 * ks) & 3) + 4 * grp;
        const int kc1 = 64 * slot + 16 * ((2 * ks + 1) & 3) + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const T* vr = &sVT[(16 * dt + col) * kVRow];
          const uint2 lo = *(const uint2*)(vr + kc0);
          const uint2 hi = *(const uint2*)(vr + kc1);
          const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bp, oacc[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int slot = kt < 4 ? prv : cur;
        const int kc = 64 * slot + 16 * (kt & 3) + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const float4 a = *(const float4*)(&sVT[(16 * dt + col) * kVRow + kc]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, acc[kt][0], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, acc[kt][1], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, acc[kt][2], oacc[dt], 0, 0, 0);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, acc[kt][3], oacc[dt], 0, 0, 0);
        }
      }
    }

    // ---- normalise and store: lane holds dims 16 dt + 4 grp + 0..3 of its query ----
    const float rs = 1.0f / sum;
    const size_t slot_g = (size_t)c * kChunk + qrow;
    T* orow = o_sorted + ((size_t)bh * n_slots + slot_g) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const float o0 = oacc[dt][0] * rs, o1 = oacc[dt][1] * rs, o2 = oacc[dt][2] * rs, o3 = oacc[dt][3] * rs;
      if constexpr (BF16) {
        const uint32_t w0 = (uint32_t)f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16_bits(o2) | ((uint32_t)f32_to_bf16_bits(o3) << 16);
        *(uint2*)(orow + 16 * dt + 4 * grp) = make_uint2(w0, w1);
      } else {
        *(float4*)(orow + 16 * dt + 4 * grp) = make_float4(o0, o1, o2, o3);
      }
    }
    if (grp == 0) lse_sorted[(size_t)bh * n_slots + slot_g] = (mx + __log2f(sum)) * kLn2;
    __syncthreads();
  }
}

template <bool BF16>
hipError_t launch_attn_t(const void* qk, const void* v, const int32_t* sorted_idx, void* o_sorted,
                         float* lse_sorted, int BH, int L, int n_h, int causal, hipStream_t s) {
  using T = typename AttnTraits<BF16>::T;
  const int n_slots = n_h * L;
  const int n_chunks = n_slots / kChunk;
  const int blocks_per_bh = (n_chunks + kChunksPerBlock - 1) / kChunksPerBlock;
  const unsigned grid = (unsigned)blocks_per_bh * (unsigned)BH;
  if (causal)
    chunk_attn_kernel<BF16, true><<<grid, 256, 0, s>>>((const T*)qk, (const T*)v, sorted_idx, (T*)o_sorted,
                                                       lse_sorted, L, n_slots, n_chunks, blocks_per_bh);
  else
    chunk_attn_kernel<BF16, false><<<grid, 256, 0, s>>>((const T*)qk, (const T*)v, sorted_idx, (T*)o_sorted,
                                                        lse_sorted, L, n_slots, n_chunks, blocks_per_bh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_attn(const void* qk, const void* v, const int32_t* sorted_idx, void* o_sorted,
                             float* lse_sorted, int BH, int L, int n_h, int causal, lsh_dtype dt,
                             hipStream_t s) {
  if (dt == LSH_BF16) return launch_attn_t<true>(qk, v, sorted_idx, o_sorted, lse_sorted, BH, L, n_h, causal, s);
  return launch_attn_t<false>(qk, v, sorted_idx, o_sorted, lse_sorted, BH, L, n_h, causal, s);
}

}  // namespace lsh
