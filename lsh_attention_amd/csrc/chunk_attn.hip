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
// gfx950 design (one block of 4 waves walks a run of 8 consecutive chunks of
// one (batch, head); wave w owns queries 16w..16w+15 of the current chunk; 128
// VGPRs and 35 KiB of LDS per block, so 4 blocks share a CU):
//  * Gathers are software-pipelined: the 64 x rows and 64 v rows of chunk c+1
//    (128-byte rows addressed through sorted_idx) are loaded into registers
//    while chunk c is computed, then written to LDS.  The previous chunk's
//    rows stay resident (two-slot ring), so each row is gathered once per
//    block.  The block's slice of sorted_idx is staged in LDS up front.
//  * V is stored transposed in LDS for the P.V product, with its keys permuted
//    into the order the P.V operand consumes them, so each lane reads its 8
//    keys as one 16-byte LDS read.  Each thread gathers one 4-byte word (two
//    dims) from each of 8 rows and writes two 16-byte V^T pieces, so the
//    transpose costs 2 LDS writes per thread per chunk.  The bf16 tiles use
//    unpadded rows with XOR-swizzled 16-byte pieces (xoff / voff below), the
//    layout that lets both the operand reads and these writes run at full rate.
//  * S^T = K Q^T on MFMA (keys are MFMA rows, queries MFMA columns), so each
//    lane holds one query's logits for 4 consecutive keys per 16-key tile.
//  * O^T = V^T P^T on MFMA: the P^T operand is exactly the lane's own
//    probabilities (the K index is permuted to match).
//  * bf16 fast path: S MFMAs, softmax and P.V MFMAs of a chunk run as one
//    interleaved stream per wave (stage kt: tile kt+1's S, tile kt's
//    probabilities, an earlier key pair's P.V), not as three serial phases.
//  * Per-row key scale and query bound come from the hash pass in the fused
//    forward (token_scales); the standalone call computes them from the rows.
//  * A query's 128 logits sit in 4 lanes (l, l^16, l^32, l^48); their sums and
//    maxima use the gfx950 permlane32/permlane16 swaps, not LDS.
//  * Softmax offset: keys are unit-normalised, so every logit is at most
//    M_i = |x_i| / sqrt(64) (Cauchy-Schwarz).  Offsetting by M_i instead of the
//    row maximum gives the same softmax and lse, needs no max reduction, and
//    the self / causal masks become one compare that zeroes the probability.
//    If a row's sum falls below 2^-60 (only a self-only row, or keys far from
//    the query's direction at huge norms), the wave recomputes that chunk with
//    the row maximum and the explicit -1e5 self logit.
#include <type_traits>

#include "lsh_internal.h"

namespace lsh {

namespace {

constexpr int kChunksPerBlock = 8;
constexpr size_t kAttnFillBlocks = 1024;  // 4 blocks on each of 256 CUs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSelf2 = -1.0e5f * kLog2e;        // self logit, base 2
constexpr float kMinSum = 0x1p-60f;               // fast-path validity threshold

template <bool BF16>
struct AttnTraits;
template <>
struct AttnTraits<true> {
  using T = uint16_t;
  static constexpr int kXRow = 64;   // x rows in LDS: 64 dims, 16-byte pieces swizzled (xoff)
  static constexpr int kVRow = 128;  // V^T rows in LDS: 2 slots x 64 keys, pieces swizzled (voff)
  static constexpr int kXLoads = 2;  // 16-byte loads per thread for its 16 dims of an x row
  static constexpr int kVWords = 8;  // 4-byte V words per thread (2 dims x 8 rows)
};
template <>
struct AttnTraits<false> {
  using T = float;
  static constexpr int kXRow = 68;
  static constexpr int kVRow = 132;
  static constexpr int kXLoads = 4;
  static constexpr int kVWords = 16;  // 1 dim x 16 rows
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

// bf16 LDS tiles keep rows unpadded and store 16-byte piece q of row r at
// piece q ^ (r mod pieces-per-row).  The MFMA operand reads (16 lanes on 16
// rows, the 4 lane groups on 4 pieces) and the staging writes then run at the
// full LDS rate on gfx950; padded rows of 144 or 272 bytes measured 1.6x slower
// for those reads.  Element offsets:
__device__ inline int xoff(int row, int piece) { return row * 64 + 8 * (piece ^ (row & 7)); }    // x rows
__device__ inline int voff(int row, int piece) { return row * 128 + 8 * (piece ^ (row & 15)); }  // V^T rows

// ATTEND: 0 = the method as described; bit 0 = same-bucket keys only, bit 1 =
// set union over the rounds (each distinct key once).  The variants take the
// exact softmax path for every chunk, walk 4 chunks per block and keep their
// per-row tables in dynamic LDS (variant_lds_bytes), so the base kernel's
// resources are unchanged.
template <int ATTEND>
constexpr int chunks_per_block() { return ATTEND ? 4 : kChunksPerBlock; }

// Dynamic LDS of a variant, as ints per sPos entry (kCPB + 1 of them) and row:
//   same-bucket: 1 code, (round << 13) | bucket;
//   set union:   n_h words, one per round r: the token's chunk index within
//                round r, or with same-bucket (bucket_r << 18) | that index;
//                plus 2 masks (last / first, below).
inline size_t variant_lds_bytes(int attend, int n_h) {
  if (attend == 0) return 0;
  const int per_row = ((attend & 1) ? 1 : 0) + ((attend & 2) ? n_h + 2 : 0);
  return (size_t)(chunks_per_block<1>() + 1) * 64 * per_row * sizeof(int);
}

// NT: the output rows are written with non-temporal stores (stream_slot_rows).
template <bool BF16, bool CAUSAL, int ATTEND, bool NT = false>
__global__ __launch_bounds__(256, (BF16 && ATTEND == 0) ? 4 : 2) void chunk_attn_kernel(
    const typename AttnTraits<BF16>::T* __restrict__ qk, const typename AttnTraits<BF16>::T* __restrict__ v,
    const int32_t* __restrict__ sorted_idx, typename AttnTraits<BF16>::T* __restrict__ o_out,
    float* __restrict__ lse_out, const float2* __restrict__ token_scales, const int32_t* __restrict__ buckets,
    const int32_t* __restrict__ tok_rec, int L, int n_h, int n_slots, int n_chunks, int blocks_per_bh, int cpb,
    int n_bh, bool xcd_local) {
  constexpr int kCPB = chunks_per_block<ATTEND>();  // the longest run (cpb <= kCPB)
  constexpr bool kSB = (ATTEND & 1) != 0, kDD = (ATTEND & 2) != 0;
  using T = typename AttnTraits<BF16>::T;
  constexpr int kXRow = AttnTraits<BF16>::kXRow;
  constexpr int kVRow = AttnTraits<BF16>::kVRow;
  constexpr int kXLoads = AttnTraits<BF16>::kXLoads;
  constexpr int kVWords = AttnTraits<BF16>::kVWords;
  __shared__ __attribute__((aligned(16))) T sX[2][64 * kXRow];
  __shared__ __attribute__((aligned(16))) T sVT[64 * kVRow];  // [dim][64 * slot + key]
  __shared__ __attribute__((aligned(16))) float sKs[2][64];   // key scale: log2(e) / (8 |x_j|)
  __shared__ __attribute__((aligned(16))) float sM[2][64];    // query bound: log2(e) |x_i| / 8
  __shared__ __attribute__((aligned(16))) int sPos[kCPB + 1][64];
  __shared__ __attribute__((aligned(16))) float sPf[kCPB + 1][64];  // 2 * position (exact below 2^23)
  // Variant tables (dynamic LDS, [entry][row] each, rounds inner for sChk):
  // sCode, sChk[entry][round][row], sLast, sFirst.
  extern __shared__ __attribute__((aligned(16))) int sVar[];
  int* const sCode = sVar;
  int* const sChk = sVar + (kSB ? (kCPB + 1) * 64 : 0);
  int* const sLast = sChk + (kDD ? (kCPB + 1) * n_h * 64 : 0);
  int* const sFirst = sLast + (kDD ? (kCPB + 1) * 64 : 0);

  // xcd_local: the runs of one (batch, head) share an XCD (consecutive items on
  // one XCD), so its gathered rows meet in one L2 instead of all eight.
  // Otherwise blocks go round-robin over the XCDs in item order, so all XCDs
  // work on the same few heads at a time.
  const unsigned item = xcd_local ? xcd_item(blockIdx.x, gridDim.x) : blockIdx.x;
  if (item >= (unsigned)blocks_per_bh * (unsigned)n_bh) return;
  const int bh = (int)item / blocks_per_bh;
  const int c0 = ((int)item % blocks_per_bh) * cpb;
  const int c1 = min(n_chunks, c0 + cpb);
  const int cpr = L / kChunk;  // chunks per round
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15;  // query (column) of the MFMA tiles
  const int grp = lane >> 4;  // 4-key group within a 16-key tile

  // Per-(b,h) bases; rows are addressed with 32-bit byte offsets (L * 64 * 4 < 2^32).
  constexpr uint32_t kRowBytes = kD * sizeof(T);
  const char* xq = (const char*)(qk + (size_t)bh * L * kD);
  const char* vq = (const char*)(v + (size_t)bh * L * kD);
  const int32_t* sidx = sorted_idx + (size_t)bh * n_slots;
  T* obase = o_out + (size_t)bh * n_slots * kD;
  float* lbase = lse_out + (size_t)bh * n_slots;

  // Positions of the previous chunk of c0 and of chunks c0..c1-1 (entry k <-> chunk c0-1+k).
  // Positions come from a permutation of [0, L); the clamp only keeps a
  // malformed index array from reading out of bounds.
  for (int e = tid; e < (c1 - c0 + 1) * 64; e += 256) {
    const int k = e >> 6, r = e & 63;
    const int c = (k == 0) ? (c0 - 1 + n_chunks) % n_chunks : c0 - 1 + k;
    const int pos = (int)min((uint32_t)sidx[(size_t)c * kChunk + r], (uint32_t)(L - 1));
    sPos[k][r] = pos;
    sPf[k][r] = 2.0f * (float)pos;
  }
  __syncthreads();
  if constexpr (ATTEND != 0) {
    const int cpr = L / kChunk;  // chunks per round
    const int32_t* bk = buckets + (size_t)bh * n_h * L;
    for (int e = tid; e < (c1 - c0 + 1) * 64; e += 256) {
      const int k = e >> 6, r = e & 63;
      const int c = (k == 0) ? (c0 - 1 + n_chunks) % n_chunks : c0 - 1 + k;
      const int pos = sPos[k][r];
      // the token's record: per round, (bucket << 18) | chunk index within the round
      const int32_t* rec = kDD ? tok_rec + ((size_t)bh * L + pos) * n_h : nullptr;
      if constexpr (kSB) {
        const int rnd = c / cpr;
        const int bucket = kDD ? rec[rnd] >> 18 : bk[(size_t)rnd * L + pos] & 0xFFF;
        sCode[k * 64 + r] = (rnd << 13) | bucket;
      }
      if constexpr (kDD) {
        int32_t wv[kMaxHashes];
#pragma unroll
        for (int b = 0; b < kMaxHashes; ++b)
          if (b < n_h) wv[b] = rec[b];
        int last = 0, first = 0;
#pragma unroll
        for (int b = 0; b < kMaxHashes; ++b)
          if (b < n_h) {
            const int cb = wv[b] & 0x3FFFF;
            sChk[(k * n_h + b) * 64 + r] = kSB ? wv[b] : cb;
            last |= (cb == cpr - 1 ? 1 : 0) << b;
            // bit b: this token's chunk in round b+1 (cyclically) is that round's first
            first |= (cb == 0 ? 1 : 0) << ((b + n_h - 1) % n_h);
          }
        sLast[k * 64 + r] = last;
        sFirst[k * 64 + r] = first;
      }
    }
    __syncthreads();
  }

  // ---- gather of one chunk into registers, and from registers into LDS ----
  // x: thread t holds 16 dims (quarter t&3) of row t>>2.
  // v: bf16: dims 2p, 2p+1 (p = t&31) of rows 8(t>>5)..+7; fp32: dim t&63 of rows 16(t>>6)..+15.
  uint4 xr[kXLoads];
  uint32_t vw[kVWords];
  float2 tsc = make_float2(0.f, 0.f);  // (key scale, query bound) of row tid, when precomputed
  const int xrow = tid >> 2, xq4 = tid & 3;
  const float2* tsq = token_scales == nullptr ? nullptr : token_scales + (size_t)bh * L;
  auto gather = [&](int k) {
    const int* pos = sPos[k];
    if (tsq != nullptr && tid < 64) tsc = tsq[pos[tid]];
    const uint32_t xoff = (uint32_t)pos[xrow] * kRowBytes + 16u * xq4 * (uint32_t)sizeof(T);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) xr[i] = *(const uint4*)(xq + xoff + 16u * i);
    if constexpr (BF16) {
      const uint32_t p4 = 4u * (tid & 31);
      const int j = tid >> 5, r0 = 32 * (j >> 2) + 4 * (j & 3);
#pragma unroll
      for (int i = 0; i < 8; ++i) vw[i] = *(const uint32_t*)(vq + ((uint32_t)pos[r0 + (i & 3) + 16 * (i >> 2)] * kRowBytes + p4));
    } else {
      const uint32_t p4 = 4u * (tid & 63);
      const int r0 = 16 * (tid >> 6);
#pragma unroll
      for (int i = 0; i < 16; ++i) vw[i] = *(const uint32_t*)(vq + ((uint32_t)pos[r0 + i] * kRowBytes + p4));
    }
  };
  auto commit = [&](int slot) {
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      if constexpr (BF16)
        *(uint4*)(&sX[slot][xoff(xrow, 2 * xq4 + i)]) = xr[i];
      else
        *(uint4*)(&sX[slot][xrow * kXRow + 16 * xq4 + i * (16 / kXLoads)]) = xr[i];
    }
    if (tsq != nullptr) {
      if (tid < 64) {
        sKs[slot][tid] = tsc.x;
        sM[slot][tid] = tsc.y;
      }
    } else {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const uint32_t w4[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (BF16) {
          const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xFFFF0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        } else {
          const float f = __uint_as_float(w4[e]);
          ss = fmaf(f, f, ss);
        }
      }
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (xq4 == 0) {
      const float2 sc = token_scale(ss);
      sKs[slot][xrow] = sc.x;
      sM[slot][xrow] = sc.y;
    }
    }
    if constexpr (BF16) {
      // V^T columns are keys in the order of the P.V operand: column 32h + 8g + 4b + e holds
      // chunk row 32h + 16b + 4g + e.  This thread holds rows 32h + 4g + e and 32h + 16 + 4g + e
      // (h, g from its index), i.e. columns 32h + 8g + 0..7: piece j of the slot.  V^T rows
      // are dims in the order 0, 2, .., 62, 1, 3, .., 63 (row p = dim 2p, row 32 + p =
      // dim 2p + 1), so the 32 lanes of a half-wave write 32 consecutive rows.
      const int p = tid & 31, j = tid >> 5;
      // low halves = dim 2p, high halves = dim 2p+1, of the 8 rows in column order
      uint4 lo, hi;
      lo.x = __builtin_amdgcn_perm(vw[1], vw[0], 0x05040100u);
      lo.y = __builtin_amdgcn_perm(vw[3], vw[2], 0x05040100u);
      lo.z = __builtin_amdgcn_perm(vw[5], vw[4], 0x05040100u);
      lo.w = __builtin_amdgcn_perm(vw[7], vw[6], 0x05040100u);
      hi.x = __builtin_amdgcn_perm(vw[1], vw[0], 0x07060302u);
      hi.y = __builtin_amdgcn_perm(vw[3], vw[2], 0x07060302u);
      hi.z = __builtin_amdgcn_perm(vw[5], vw[4], 0x07060302u);
      hi.w = __builtin_amdgcn_perm(vw[7], vw[6], 0x07060302u);
      *(uint4*)(&sVT[voff(p, 8 * slot + j)]) = lo;
      *(uint4*)(&sVT[voff(32 + p, 8 * slot + j)]) = hi;
    } else {
      const int p = tid & 63, r0 = 16 * (tid >> 6);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(uint4*)(&sVT[p * kVRow + 64 * slot + r0 + 4 * i]) =
            make_uint4(vw[4 * i], vw[4 * i + 1], vw[4 * i + 2], vw[4 * i + 3]);
    }
  };

  gather(0);
  commit((c0 + 1) & 1);
  gather(1);
  commit(c0 & 1);
  __syncthreads();

  // Sum / max over the 4 lanes holding one query (lanes l, l^16, l^32, l^48)
  // with the gfx950 cross-lane swaps (no LDS round trip).
  auto qsum = [](float x) {
    auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
  };
  auto qmax = [](float x) {
    auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
    auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
  };

  for (int c = c0; c < c1; ++c) {
    const int cur = c & 1, prv = cur ^ 1;
    const int kc = c - c0 + 1;  // sPos entry of chunk c
    if (c + 1 < c1) gather(kc + 1);
    __builtin_amdgcn_s_setprio(0);

    const int qrow = 16 * wave + col;  // this lane's query row in the current chunk
    const int qpos = sPos[kc][qrow];
    const float M2 = sM[cur][qrow];

    // ---- S^T = K Q^T : 8 key tiles of 16 (tiles 0-3 previous chunk, 4-7 current) ----
    auto scores = [&](f32x4 (&acc)[8]) {
      if constexpr (BF16) {
        const bf16x8 bq0 = *(const bf16x8*)(&sX[cur][xoff(qrow, grp)]);
        const bf16x8 bq1 = *(const bf16x8*)(&sX[cur][xoff(qrow, 4 + grp)]);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          const T* kx = sX[kt < 4 ? prv : cur];
          const int krow = 16 * (kt & 3) + col;
          const bf16x8 a0 = *(const bf16x8*)(kx + xoff(krow, grp));
          const bf16x8 a1 = *(const bf16x8*)(kx + xoff(krow, 4 + grp));
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bq0, z, 0, 0, 0);
          acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bq1, z, 0, 0, 0);
        }
      } else {
        // k-step s of 4 dims: lane group g feeds dim 16g + s.
        float bq[16];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float4 t = *(const float4*)(&sX[cur][qrow * kXRow + 16 * grp + 4 * s4]);
          bq[4 * s4] = t.x;
          bq[4 * s4 + 1] = t.y;
          bq[4 * s4 + 2] = t.z;
          bq[4 * s4 + 3] = t.w;
        }
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          const T* kr = &sX[kt < 4 ? prv : cur][(16 * (kt & 3) + col) * kXRow + 16 * grp];
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
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
    };

    // ---- O^T = V^T P^T ----
    auto pv = [&](const float (&p)[8][4], f32x4 (&oacc)[4]) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // K index (grp, e): e < 4 -> key 4 grp + e of tile 2ks; e >= 4 -> of tile 2ks + 1.
          const f32x4 lo = {p[2 * ks][0], p[2 * ks][1], p[2 * ks][2], p[2 * ks][3]};
          const f32x4 hi = {p[2 * ks + 1][0], p[2 * ks + 1][1], p[2 * ks + 1][2], p[2 * ks + 1][3]};
          const bf16x4 blo = __builtin_convertvector(lo, bf16x4);
          const bf16x4 bhi = __builtin_convertvector(hi, bf16x4);
          const bf16x8 bp = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
          const int slot = ks < 2 ? prv : cur;
          // keys of tiles 2ks and 2ks+1 seen by lane group grp: V^T columns 32 (ks & 1) + 8 grp + 0..7
          const int vpiece = 8 * slot + 4 * (ks & 1) + grp;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const bf16x8 a = *(const bf16x8*)(&sVT[voff(16 * dt + col, vpiece)]);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp, oacc[dt], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          const int slot = kt < 4 ? prv : cur;
          const int kcol = 64 * slot + 16 * (kt & 3) + 4 * grp;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const float4 a = *(const float4*)(&sVT[(16 * dt + col) * kVRow + kcol]);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, p[kt][0], oacc[dt], 0, 0, 0);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, p[kt][1], oacc[dt], 0, 0, 0);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, p[kt][2], oacc[dt], 0, 0, 0);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, p[kt][3], oacc[dt], 0, 0, 0);
          }
        }
      }
    };

    f32x4 acc[8];
    float p[8][4];
    float sum = 0.f;
    f32x4 oacc[4];
    float off = M2;
    bool self_only = false, patch = false;
    if constexpr (ATTEND == 0) {
    // ---- fast path: probabilities offset by the a-priori bound M2, masks as zeroes ----
    // The causal mask is a median: y = 2 (query position - key position) is >= 2
    // for a key that is kept and <= 0 for one at or after the query, and the
    // probability is at most 1 + 2^-20, so med3(p, 0, y) is p or 0 (no
    // compare/select pair, whose mask register costs wait states between the two).
      const float qf2 = sPf[kc][qrow];
      if constexpr (BF16) {
        // One stream per wave: the offset M2 is known before any logit, so key
        // tile kt's probabilities need nothing from other tiles and the three
        // phases interleave.  Stage kt issues the two S MFMAs of tile kt+1 and
        // two P.V MFMAs of an earlier key pair next to the logits of tile kt
        // (exp, mask, sum); sched_group_barrier asks for six VALU instructions
        // after each MFMA and leaves their choice to the scheduler (pinning one
        // logit per MFMA serialises each exp chain and measured 30 % slower).
        // The LDS operands of tile kt+2 and of the next pair's V^T are read a
        // stage ahead.  The sums and the P.V accumulation keep the order of the
        // phase-by-phase form, so the results are the same bits.
        // Without the causal mask only the self key is masked.  In the current chunk
        // the query's token occurs once, at the query's own slot (tile 4 + wave,
        // key col of it), so that mask is static; the look-back chunk can hold
        // the token only when it is the previous round's last chunk (the query's
        // chunk is a round's first, c % cpr == 0, which includes a single chunk
        // looking back at itself): only then are positions compared (kLB).
        auto run_stream = [&](auto kLB) {
          const bf16x8 bq0 = *(const bf16x8*)(&sX[cur][xoff(qrow, grp)]);
          const bf16x8 bq1 = *(const bf16x8*)(&sX[cur][xoff(qrow, 4 + grp)]);
          bf16x8 ka0[8], ka1[8], va[4][4], bp[4];
          float ksv[8][4], kfv[8][4];
          int kpv[8][4];
          auto loads = [&](int kt) {
            const int slot = kt < 4 ? prv : cur;
            const T* kx = sX[slot];
            const int krow = 16 * (kt & 3) + col, kr0 = 16 * (kt & 3) + 4 * grp;
            ka0[kt] = *(const bf16x8*)(kx + xoff(krow, grp));
            ka1[kt] = *(const bf16x8*)(kx + xoff(krow, 4 + grp));
            const float4 ks = *(const float4*)(&sKs[slot][kr0]);
            ksv[kt][0] = ks.x; ksv[kt][1] = ks.y; ksv[kt][2] = ks.z; ksv[kt][3] = ks.w;
            if constexpr (CAUSAL) {
              const float4 kf = *(const float4*)(&sPf[kt < 4 ? kc - 1 : kc][kr0]);
              kfv[kt][0] = kf.x; kfv[kt][1] = kf.y; kfv[kt][2] = kf.z; kfv[kt][3] = kf.w;
            } else if (decltype(kLB)::value && kt < 4) {
              const int4 kp = *(const int4*)(&sPos[kc - 1][kr0]);
              kpv[kt][0] = kp.x; kpv[kt][1] = kp.y; kpv[kt][2] = kp.z; kpv[kt][3] = kp.w;
            }
          };
          auto vloads = [&](int ks) {
            const int vpiece = 8 * (ks < 2 ? prv : cur) + 4 * (ks & 1) + grp;
  #pragma unroll
            for (int dt = 0; dt < 4; ++dt) va[ks][dt] = *(const bf16x8*)(&sVT[voff(16 * dt + col, vpiece)]);
          };
          auto smfma = [&](int kt, int h) {
            if (h == 0)
              acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0[kt], bq0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1[kt], bq1, acc[kt], 0, 0, 0);
          };
          auto pvm = [&](int ks, int dt) {
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ks][dt], bp[ks], oacc[dt], 0, 0, 0);
          };
          auto soft = [&](int kt, int e) {
            const float q = __builtin_amdgcn_exp2f(fmaf(acc[kt][e], ksv[kt][e], -M2));
            if constexpr (CAUSAL)
              p[kt][e] = __builtin_amdgcn_fmed3f(q, 0.f, qf2 - kfv[kt][e]);
            else if (kt >= 4)  // the current chunk holds the token once: its own slot
              p[kt][e] = (kt - 4 == wave && 4 * grp + e == col) ? 0.f : q;
            else if constexpr (decltype(kLB)::value)
              p[kt][e] = kpv[kt][e] == qpos ? 0.f : q;
            else
              p[kt][e] = q;
            sum += p[kt][e];
          };
  #pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          loads(0);
          loads(1);
          smfma(0, 0);
          smfma(0, 1);
          loads(2);
  #pragma unroll
          for (int kt = 0; kt < 8; ++kt) {
            // P.V of key pair (kt - 2) / 2, dims 2 (kt & 1) + 0, 1: its probabilities
            // were packed and its V^T operands read in stage kt - 1 or earlier.
            const bool pv_here = kt >= 2;
            const int ks = (kt - 2) >> 1, dt0 = 2 * (kt & 1);
            if (kt + 1 < 8) smfma(kt + 1, 0);
            soft(kt, 0);
            if (pv_here) pvm(ks, dt0);
            soft(kt, 1);
            if (kt + 1 < 8) smfma(kt + 1, 1);
            soft(kt, 2);
            if (pv_here) pvm(ks, dt0 + 1);
            soft(kt, 3);
            if (kt + 2 < 8) loads(kt + 2);
            if (kt & 1) {
              // K index (grp, e): e < 4 -> key 4 grp + e of tile kt - 1; e >= 4 -> of tile kt.
              const f32x4 lo = {p[kt - 1][0], p[kt - 1][1], p[kt - 1][2], p[kt - 1][3]};
              const f32x4 hi = {p[kt][0], p[kt][1], p[kt][2], p[kt][3]};
              bp[kt >> 1] = __builtin_shufflevector(__builtin_convertvector(lo, bf16x4),
                                                    __builtin_convertvector(hi, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
              vloads(kt >> 1);
            }
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            }
          }
          sum = qsum(sum);
  #pragma unroll
          for (int dt = 0; dt < 4; ++dt) pvm(3, dt);
        };
        if constexpr (CAUSAL)
          run_stream(std::false_type{});
        else if (c % cpr == 0)
          run_stream(std::true_type{});
        else
          run_stream(std::false_type{});
      } else {
      scores(acc);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int slot = kt < 4 ? prv : cur;
        const int kr0 = 16 * (kt & 3) + 4 * grp;
        const float4 ks = *(const float4*)(&sKs[slot][kr0]);
        const float ksv[4] = {ks.x, ks.y, ks.z, ks.w};
        if constexpr (CAUSAL) {
          const float4 kf = *(const float4*)(&sPf[kt < 4 ? kc - 1 : kc][kr0]);
          const float kfv[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float q = __builtin_amdgcn_exp2f(fmaf(acc[kt][e], ksv[e], -M2));
            p[kt][e] = __builtin_amdgcn_fmed3f(q, 0.f, qf2 - kfv[e]);
            sum += p[kt][e];
          }
        } else {
          // only the self key is masked
          const int4 kp = *(const int4*)(&sPos[kt < 4 ? kc - 1 : kc][kr0]);
          const int kpos[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float q = __builtin_amdgcn_exp2f(fmaf(acc[kt][e], ksv[e], -M2));
            p[kt][e] = kpos[e] == qpos ? 0.f : q;
            sum += p[kt][e];
          }
        }
      }
      sum = qsum(sum);
      pv(p, oacc);
      }
      // A row whose sum is not usable.  With M2 < 60 every kept key has probability
      // at least 2^-120, so a zero sum means that every key but the self was masked.
      // In a chunk that is not the first of its round the look-back chunk belongs
      // to the same round, so the self key occurs once and the exact result is
      // o = v_self, lse = -1e5: such rows are patched after the normalisation (the
      // common rare case: causal queries early in the sequence).  Anything else (a
      // self key that may occur twice, a tiny non-zero sum) takes the exact path.
      const bool z = !(sum >= kMinSum);
      self_only = z && sum == 0.f && M2 < 60.f;
      if (__builtin_expect(__ballot(z) != 0ull, 0))
        patch = (c % cpr) != 0 && __ballot(z && !self_only) == 0ull;
      if (__builtin_expect(__ballot(z && !patch) != 0ull, 0)) {
        // Exact path for the wave (rare): logits with the -1e5 self value and the
        // row maximum, recomputed from the LDS tiles.  The clobber makes this path
        // reload its LDS operands instead of keeping the fast path's loads live.
        asm volatile("" ::: "memory");
        scores(acc);
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          const int slot = kt < 4 ? prv : cur;
          const int kr0 = 16 * (kt & 3) + 4 * grp;
          const float4 ks = *(const float4*)(&sKs[slot][kr0]);
          const int4 kp = *(const int4*)(&sPos[kt < 4 ? kc - 1 : kc][kr0]);
          const float ksv[4] = {ks.x, ks.y, ks.z, ks.w};
          const int kpos[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sc = acc[kt][e] * ksv[e];
            if (kpos[e] == qpos) sc = kSelf2;
            if (CAUSAL && kpos[e] > qpos) sc = -INFINITY;
            p[kt][e] = sc;
            mx = fmaxf(mx, sc);
          }
        }
        mx = qmax(mx);
        sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[kt][e] = __builtin_amdgcn_exp2f(p[kt][e] - mx);
            sum += p[kt][e];
          }
        sum = qsum(sum);
        off = mx;
        pv(p, oacc);
      }
    } else {
      // ---- attended-set variants: exact path (row maximum) for every chunk ----
      scores(acc);
      // same-bucket: keys with another (round, bucket) code than the query are
      // dropped.  set union: each kept logit, the self's included, gets
      // -log2 N, N = the number of (query occurrence, key occurrence) pairs of
      // the token pair over all rounds' windows:
      //   N = sum_r [0 <= chunk_r(query) - chunk_r(key) <= 1]   (the window of
      //         the query's round-r chunk; with same-bucket only if the two
      //         share the round-r bucket: the packed words differ by 0 or 1)
      //     + #{r : the key's round-r chunk is that round's last and the
      //         query's round-(r+1) chunk is that round's first}   (the look-back
      //         across a round boundary; with same-bucket it joins one round's
      //         ends, so only for n_h == 1 and equal buckets).
      int nn[8][4];
      if constexpr (kDD) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) nn[kt][e] = 0;
        for (int b = 0; b < n_h; ++b) {
          const int qw = sChk[(kc * n_h + b) * 64 + qrow];
#pragma unroll
          for (int kt = 0; kt < 8; ++kt) {
            const int ke = kt < 4 ? kc - 1 : kc;
            const int4 w4 = *(const int4*)(&sChk[(ke * n_h + b) * 64 + 16 * (kt & 3) + 4 * grp]);
            nn[kt][0] += (uint32_t)(qw - w4.x) <= 1u ? 1 : 0;
            nn[kt][1] += (uint32_t)(qw - w4.y) <= 1u ? 1 : 0;
            nn[kt][2] += (uint32_t)(qw - w4.z) <= 1u ? 1 : 0;
            nn[kt][3] += (uint32_t)(qw - w4.w) <= 1u ? 1 : 0;
          }
        }
        if (!kSB || n_h == 1) {
          const int qf = sFirst[kc * 64 + qrow];
          const int qb = sChk[kc * n_h * 64 + qrow] >> 18;  // round-0 bucket (same-bucket only)
#pragma unroll
          for (int kt = 0; kt < 8; ++kt) {
            const int ke = kt < 4 ? kc - 1 : kc;
            const int kr0 = 16 * (kt & 3) + 4 * grp;
            const int4 l4 = *(const int4*)(&sLast[ke * 64 + kr0]);
            const int kl[4] = {l4.x, l4.y, l4.z, l4.w};
            int same[4] = {1, 1, 1, 1};
            if constexpr (kSB) {
              const int4 w4 = *(const int4*)(&sChk[ke * n_h * 64 + kr0]);
              same[0] = (w4.x >> 18) == qb; same[1] = (w4.y >> 18) == qb;
              same[2] = (w4.z >> 18) == qb; same[3] = (w4.w >> 18) == qb;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) nn[kt][e] += same[e] ? __popc((uint32_t)(kl[e] & qf)) : 0;
          }
        }
      }
      const int qcode = kSB ? sCode[kc * 64 + qrow] : 0;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int ke = kt < 4 ? kc - 1 : kc;
        const int slot = kt < 4 ? prv : cur;
        const int kr0 = 16 * (kt & 3) + 4 * grp;
        const float4 ks = *(const float4*)(&sKs[slot][kr0]);
        const int4 kp = *(const int4*)(&sPos[ke][kr0]);
        const float ksv[4] = {ks.x, ks.y, ks.z, ks.w};
        const int kpos[4] = {kp.x, kp.y, kp.z, kp.w};
        int kcode[4] = {0, 0, 0, 0};
        if constexpr (kSB) {
          const int4 c4 = *(const int4*)(&sCode[ke * 64 + kr0]);
          kcode[0] = c4.x; kcode[1] = c4.y; kcode[2] = c4.z; kcode[3] = c4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sc = acc[kt][e] * ksv[e];
          if (kpos[e] == qpos) sc = kSelf2;
          if (CAUSAL && kpos[e] > qpos) sc = -INFINITY;
          if (kSB && kcode[e] != qcode) sc = -INFINITY;
          if (kDD && nn[kt][e] > 1) sc -= __builtin_amdgcn_logf((float)nn[kt][e]);  // log2
          p[kt][e] = sc;
          mx = fmaxf(mx, sc);
        }
      }
      mx = qmax(mx);
#pragma unroll
      for (int kt = 0; kt < 8; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[kt][e] = __builtin_amdgcn_exp2f(p[kt][e] - mx);
          sum += p[kt][e];
        }
      sum = qsum(sum);
      off = mx;
      pv(p, oacc);
    }

    // ---- normalise and store ----
    const float rs = __builtin_amdgcn_rcpf(sum);
    const size_t row_g = (size_t)c * kChunk + qrow;
    T* orow = obase + row_g * kD;
    const bool own = patch && self_only;  // o = v_self, lse = -1e5
    uint32_t ow[BF16 ? 8 : 16];           // the lane's pieces of the output row
    const char* vself = vq + (uint32_t)qpos * kRowBytes;
    if constexpr (BF16) {
      // O^T row r is V^T row r: dim 2r for r < 32, dim 2(r - 32) + 1 above.  The
      // lane's tiles 0 and 2 hold dims 8 grp + 0..7 (even, odd interleaved), tiles
      // 1 and 3 dims 32 + 8 grp + 0..7: two 16-byte pieces of the output row.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ow[4 * h + e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                           f32x2{oacc[h][e] * rs, oacc[h + 2][e] * rs}, bf16x2));
      if (__builtin_expect(own, 0)) {
        const uint4 a = *(const uint4*)(vself + 16u * grp), b = *(const uint4*)(vself + 64u + 16u * grp);
        ow[0] = a.x; ow[1] = a.y; ow[2] = a.z; ow[3] = a.w;
        ow[4] = b.x; ow[5] = b.y; ow[6] = b.z; ow[7] = b.w;
      }
    } else {
      // lane holds dims 16 dt + 4 grp + 0..3 of its query
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) ow[4 * dt + e] = __float_as_uint(oacc[dt][e] * rs);
      if (__builtin_expect(own, 0)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint4 a = *(const uint4*)(vself + 4u * (16 * dt + 4 * grp));
          ow[4 * dt] = a.x; ow[4 * dt + 1] = a.y; ow[4 * dt + 2] = a.z; ow[4 * dt + 3] = a.w;
        }
      }
    }
    {
      // the lane's 16-byte pieces: BF16 two (dims 8 grp.. and 32 + 8 grp..), fp32 four
      constexpr int kPc = BF16 ? 2 : 4;
#pragma unroll
      for (int h = 0; h < kPc; ++h) {
        const u32x4 piece = {ow[4 * h], ow[4 * h + 1], ow[4 * h + 2], ow[4 * h + 3]};
        u32x4* dst = (u32x4*)(orow + (BF16 ? 32 * h + 8 * grp : 16 * h + 4 * grp));
        if constexpr (NT)
          __builtin_nontemporal_store(piece, dst);
        else
          *dst = piece;
      }
    }
    if (grp == 0) lbase[row_g] = own ? kSelf2 * kLn2 : (off + __builtin_amdgcn_logf(sum)) * kLn2;

    // From here through the issue of the next iteration's gather the wave runs
    // at raised priority: the block's critical path (the barriers, the commit
    // to LDS, the next loads) goes ahead of the other blocks' vector work on
    // the SIMD (measured: about 2 us of 324 at long_seq_64k).
    __builtin_amdgcn_s_setprio(2);
    __syncthreads();  // every wave is done with slot prv
    if (c + 1 < c1) {
      commit(prv);
      __syncthreads();
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Token-major record of the set-union variant: rec[bh][i][r] = (bucket of i in
// round r << 18, 0 without buckets) | (chunk of i in round r, as an index within
// the round).  One
// contiguous n_h-word record per token, so the attention kernel reads a row's
// rounds as one sector instead of 2 n_h scattered words.  Undo values of round
// r lie in [r L, (r+1) L); out-of-range values only give wrong table data.
__global__ __launch_bounds__(256) void variant_rec_kernel(const int32_t* __restrict__ buckets,
                                                          const int32_t* __restrict__ undo_idx,
                                                          int32_t* __restrict__ rec, int L, int n_h,
                                                          int blocks_per_bh) {
  const int bh = blockIdx.x / blocks_per_bh;
  const int i = (blockIdx.x % blocks_per_bh) * 256 + threadIdx.x;
  if (i >= L) return;
  const int cpr = L / kChunk;
  const int32_t* ud = undo_idx + (size_t)bh * n_h * L;
  int32_t* out = rec + ((size_t)bh * L + i) * n_h;
  for (int r = 0; r < n_h; ++r) {
    const int cb = (ud[(size_t)r * L + i] >> 6) - r * cpr;
    const int bucket = buckets == nullptr ? 0 : buckets[((size_t)bh * n_h + r) * L + i] & 0xFFF;
    out[r] = (bucket << 18) | (cb & 0x3FFFF);
  }
}

template <bool BF16, int ATTEND>
hipError_t launch_attn_t(const void* qk, const void* v, const int32_t* sorted_idx, void* o_out, float* lse_out,
                         const float2* token_scales, const int32_t* buckets, const int32_t* tok_rec, int BH,
                         int L, int n_h, int causal, hipStream_t s) {
  using T = typename AttnTraits<BF16>::T;
  constexpr int kCPB = chunks_per_block<ATTEND>();
  const int n_slots = n_h * L;
  const int n_chunks = n_slots / kChunk;
  // Runs of kCPB chunks, halved while the launch would not give every CU four
  // blocks (small problems: more, shorter runs, each re-gathering its look-back
  // chunk, instead of a few long serial walks).
  int cpb = kCPB;
  while (cpb > 1 && (size_t)BH * (size_t)((n_chunks + cpb - 1) / cpb) < kAttnFillBlocks) cpb >>= 1;
  const int blocks_per_bh = (n_chunks + cpb - 1) / cpb;
  // A (batch, head)'s QK and V rows are gathered again in every round.  When
  // they fit one XCD's L2 (4 MiB), keeping each head's runs on one XCD turns
  // those re-gathers into L2 hits (causal_lm_4k 79 -> 73 us, peaked_vmf_16k
  // 278 -> 265 us); when they do not (16.8 MB per head at L 65536), spreading
  // the blocks in order keeps all XCDs on the same heads, which the shared
  // last-level cache serves better (284 -> 278 us).
  const bool xcd_local = 2ull * (unsigned long long)L * kD * sizeof(T) <= (4ull << 20);
  const unsigned n_items = (unsigned)blocks_per_bh * (unsigned)BH;
  const unsigned grid = xcd_local ? xcd_grid(n_items) : n_items;
  const size_t dyn = variant_lds_bytes(ATTEND, n_h);
  // the base bf16 kernel streams large outputs past the last-level cache
  const bool nt = BF16 && ATTEND == 0 && stream_slot_rows(BH, L, n_h, BF16 ? LSH_BF16 : LSH_F32);
  auto go = [&](auto causal_tag, auto nt_tag) {
    chunk_attn_kernel<BF16, decltype(causal_tag)::value, ATTEND, decltype(nt_tag)::value><<<grid, 256, dyn, s>>>(
        (const T*)qk, (const T*)v, sorted_idx, (T*)o_out, lse_out, token_scales, buckets, tok_rec, L, n_h,
        n_slots, n_chunks, blocks_per_bh, cpb, BH, xcd_local);
  };
  using True = std::true_type;
  using False = std::false_type;
  if constexpr (BF16 && ATTEND == 0) {
    if (causal)
      nt ? go(True{}, True{}) : go(True{}, False{});
    else
      nt ? go(False{}, True{}) : go(False{}, False{});
  } else {
    if (causal)
      go(True{}, False{});
    else
      go(False{}, False{});
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_attn_d(const void* qk, const void* v, const int32_t* sorted_idx, void* o_out, float* lse_out,
                         const float2* token_scales, const int32_t* buckets, const int32_t* tok_rec, int BH,
                         int L, int n_h, int causal, int attend, hipStream_t s) {
  switch (attend) {
    case 0:
      return launch_attn_t<BF16, 0>(qk, v, sorted_idx, o_out, lse_out, token_scales, nullptr, nullptr, BH, L, n_h,
                                    causal, s);
    case 1:
      return launch_attn_t<BF16, 1>(qk, v, sorted_idx, o_out, lse_out, token_scales, buckets, nullptr, BH, L, n_h,
                                    causal, s);
    case 2:
      return launch_attn_t<BF16, 2>(qk, v, sorted_idx, o_out, lse_out, token_scales, nullptr, tok_rec, BH, L, n_h,
                                    causal, s);
    case 3:
      return launch_attn_t<BF16, 3>(qk, v, sorted_idx, o_out, lse_out, token_scales, nullptr, tok_rec, BH, L, n_h,
                                    causal, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_chunk_attn(const void* qk, const void* v, const int32_t* sorted_idx, void* o_out,
                             float* lse_out, const float2* token_scales, const int32_t* buckets,
                             const int32_t* undo_idx, int32_t* tok_rec, int BH, int L, int n_h, int causal,
                             int attend, lsh_dtype dt, hipStream_t s) {
  if (attend & 2) {
    const int blocks_per_bh = (L + 255) / 256;
    variant_rec_kernel<<<(unsigned)blocks_per_bh * (unsigned)BH, 256, 0, s>>>(buckets, undo_idx, tok_rec, L, n_h,
                                                                             blocks_per_bh);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dt == LSH_BF16)
    return launch_attn_d<true>(qk, v, sorted_idx, o_out, lse_out, token_scales, buckets, tok_rec, BH, L, n_h,
                               causal, attend, s);
  return launch_attn_d<false>(qk, v, sorted_idx, o_out, lse_out, token_scales, buckets, tok_rec, BH, L, n_h,
                              causal, attend, s);
}

}  // namespace lsh
