// Step 1 of the shared-QK LSH attention forward pass: angular LSH.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer), angular-LSH
// passage: a token's bucket is the angular sector its vector falls in after a
// random rotation, one independent rotation per hash round.  Concretely the
// bucket is the index of the largest entry of [x R_r ; -x R_r], lowest index
// on exact ties, with R_r of shape [D, n_b/2].
//
// gfx950 design:
//  * The projection x R_r is a dense contraction (K = 64), done on MFMA with
//    the rotation as the A operand (rotation columns = MFMA rows) and the
//    tokens as the B operand (tokens = MFMA columns), so each lane's
//    accumulators hold one token's scores for 16 rotation columns.
//  * The argmax is fused into the MFMA epilogue.  Each score becomes a sort
//    key: |score| with its low mantissa bits replaced by a column code; the
//    running top-2 keys are kept per lane with max3/med3 (2.25 VALU
//    instructions per score; on gfx950 MFMA and VALU time add up, so the
//    VALU count per score is what matters).  The winner's index comes from its
//    code, its sign from one recomputed dot product per token-round.
//  * The decision is certified: an fp32 sum of 64 exact bf16 products (or
//    rounded fp32 products) is within eps = 65 * 2^-23 * |x| * max_j |r_j| of
//    the exact value, and the key truncation adds at most one key-grid step
//    delta.  If the top-2 gap is not above 2 eps + delta the token is queued
//    for `fixup_kernel`, which re-scores the columns that may win in float64
//    (each product exact) with a rounding bound of its own, and decides the
//    ones that bound cannot separate, and the sign of a winner whose sum lies
//    within it of zero, by exact summation of the products (floating-point
//    expansions).  The result is the exact-arithmetic argmax for all finite
//    inputs whose products stay within float64's range.
//  * The rotation is shared by every (batch, head): it is transposed once per
//    call into [n_h][n_b/2 padded to 64][D] so a workgroup stages it into LDS
//    in blocks of 128 columns (64 where the padded width is not a multiple of
//    128), double-buffered with one barrier per block, and read by all four
//    waves.  bf16: the next block goes from memory straight into the free
//    buffer (global_load_lds, 16 bytes per lane, no registers) while the
//    current one is used, into XOR-swizzled 128-byte rows.  fp32: it is moved
//    in 64-column parts through registers, each part stored between two
//    pipeline steps.
//  * Each wave runs a software pipeline over 32-column tiles: the MFMAs of
//    tile t+1 are issued before the vector top-2 selection of tile t, so the
//    matrix and vector work of a wave overlap (they hardly overlap across
//    waves on gfx950).
#include "exact_sum.h"
#include "lsh_internal.h"

namespace lsh {

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline double to_f64(uint16_t b) { return (double)bf16_to_f32(b); }
__device__ inline double to_f64(float f) { return (double)f; }

__device__ inline uint32_t umax3(uint32_t a, uint32_t b, uint32_t c) {
  return max(max(a, b), c);
}
__device__ inline uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ---------------------------------------------------------------------------
// Rotation transpose [n_h][D][half] -> [n_h][halfp][D] (zero padded), the
// largest column norm of each 64-column block, and the reset of the
// uncertified-token count.  Block = (round, 64-column block).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prep_kernel(const T* __restrict__ rot, T* __restrict__ rot_t,
                                                   float* __restrict__ colmax, int* __restrict__ fix_count,
                                                   int half, int halfp, int nblk) {
  constexpr int kPer = 16 / sizeof(T);  // elements per 16-byte piece
  constexpr int kPieces = kD / kPer;    // pieces per transposed row
  __shared__ T tile[kD][65];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x / nblk, blk = blockIdx.x % nblk, j0 = blk * 64;
  const T* R = rot + (size_t)r * kD * half;
  // 64 x 64 elements, 16 per thread (column tid % 64, rows tid / 64 + 4 k), all
  // loads issued before the first is used.
  const int jj = tid & 63, d0 = tid >> 6;
  const bool in = j0 + jj < half;
  T v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = in ? R[(size_t)(d0 + 4 * k) * half + j0 + jj] : T(0);
#pragma unroll
  for (int k = 0; k < 16; ++k) tile[d0 + 4 * k][jj] = v[k];
  __syncthreads();
  // Transposed rows written as 16-byte pieces, consecutive threads on
  // consecutive pieces.
  T* RT = rot_t + ((size_t)r * halfp + j0) * kD;
#pragma unroll
  for (int k = 0; k < 64 * kPieces / 256; ++k) {
    const int q = tid + 256 * k, row = q / kPieces, pc = q % kPieces;
    union {
      T e[kPer];
      uint4 u;
    } piece;
#pragma unroll
    for (int i = 0; i < kPer; ++i) piece.e[i] = tile[kPer * pc + i][row];
    if (j0 + row < halfp) *(uint4*)(RT + (size_t)row * kD + kPer * pc) = piece.u;
  }
  // Column norms in float64, four threads per column (16 rows each), then the
  // block's largest.
  const int c = tid >> 2, q4 = tid & 3;
  double na = 0.0, nb = 0.0;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const double f = to_f64(tile[16 * q4 + i][c]), g = to_f64(tile[16 * q4 + i + 1][c]);
    na = fma(f, f, na);
    nb = fma(g, g, nb);
  }
  double nrm = na + nb;
  nrm += __shfl_xor(nrm, 1);
  nrm += __shfl_xor(nrm, 2);
  for (int off = 4; off <= 32; off <<= 1) nrm = fmax(nrm, __shfl_xor(nrm, off));
  if ((tid & 63) == 0) red[tid >> 6] = nrm;
  __syncthreads();
  if (tid == 0) {
    // Rounded up, so it bounds every column norm of the block.
    colmax[blockIdx.x] = (float)(sqrt(fmax(fmax(red[0], red[1]), fmax(red[2], red[3]))) * (1.0 + 1e-6));
    if (blockIdx.x == 0) *fix_count = 0;
  }
}

// ---------------------------------------------------------------------------
// Hash kernel.  Block = 4 waves, 64 tokens per wave (two 32-token MFMA column
// groups), 256 tokens per block; grid = (ceil(L / 256), B*H).
// ---------------------------------------------------------------------------
constexpr int kHashTok = 256;

template <bool BF16>
struct HashTraits;
template <>
struct HashTraits<true> {
  using T = uint16_t;
  // Unpadded 128-byte LDS rows whose 16-byte piece p of row r sits at
  // p ^ (r & 7) ^ ((r >> 3) & 1) (conflict-free b128 operand reads), written by
  // direct global-to-LDS loads.
  static constexpr int kRow = 64;
};
template <>
struct HashTraits<false> {
  using T = float;
  static constexpr int kRow = 68;  // 272 B
};

// CB: rotation columns staged in LDS per pass (a multiple of 64: an even number
// of 32-column tiles), one barrier per pass.
template <bool BF16, int CB>
__global__ __launch_bounds__(256, 3) void hash_kernel(const typename HashTraits<BF16>::T* __restrict__ qk,
                                                   const typename HashTraits<BF16>::T* __restrict__ rot_t,
                                                   const float* __restrict__ colmax,
                                                   int32_t* __restrict__ buckets, int* __restrict__ fix_queue,
                                                   int* __restrict__ fix_count, float2* __restrict__ token_scales,
                                                   int L, int n_h, int half, int halfp, uint32_t lowmask,
                                                   int ibits) {
  using T = typename HashTraits<BF16>::T;
  constexpr int kRow = HashTraits<BF16>::kRow;
  // Double buffer of staged rotation blocks: two arrays, so that at every use
  // the compiler knows which one a direct load writes and which one is read.
  __shared__ __attribute__((aligned(16))) T sR0[CB * kRow];
  __shared__ __attribute__((aligned(16))) T sR1[CB * kRow];
  __shared__ uint32_t sRho[kMaxHashes];  // per round: largest column norm (fp32 bits, >= 0)

  const int blocks_per_bh = (L + kHashTok - 1) / kHashTok;
  const int bh = blockIdx.x / blocks_per_bh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 31;    // token column within a 32-token group / rotation row within a tile
  const int hb = lane >> 5;   // which half of the K slice this lane feeds
  const int tok_base = (blockIdx.x % blocks_per_bh) * kHashTok + wave * 64;
  const bool wave_valid = tok_base < L;  // L % 64 == 0: a wave is all-valid or all-invalid
  const uint32_t kmask = 0x7FFFFFFFu & ~lowmask;
  // The key mask lives in a VGPR so that key = (score & mask) | code is a single
  // v_and_or_b32 with the (wave-uniform) code as its one scalar operand.
  uint32_t kmask_v;
  asm("v_mov_b32 %0, %1" : "=v"(kmask_v) : "s"(kmask));

  // B operand (tokens), kept in registers for every round.
  //  bf16: k-step s covers dims 16s..16s+15; this lane holds dims 16s + 8hb + 0..7.
  //  fp32: k-step s covers dims {s, s+32}; this lane holds dim s + 32hb.
  bf16x8 bq16[2][4];
  float bq32[2][BF16 ? 1 : 32];
  float nrm2[2];
  for (int q = 0; q < 2; ++q) {
    const int tok = tok_base + 32 * q + n;
    const T* xr = qk + ((size_t)bh * L + (wave_valid ? tok : 0)) * kD;
    float acc = 0.f;
    if constexpr (BF16) {
      for (int s = 0; s < 4; ++s) {
        uint4 raw = wave_valid ? *(const uint4*)(xr + 16 * s + 8 * hb) : make_uint4(0, 0, 0, 0);
        bq16[q][s] = __builtin_bit_cast(bf16x8, raw);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        for (int e = 0; e < 4; ++e) {
          float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xFFFF0000u);
          acc = fmaf(lo, lo, acc);
          acc = fmaf(hi, hi, acc);
        }
      }
    } else {
      for (int s4 = 0; s4 < 8; ++s4) {
        float4 raw = wave_valid ? *(const float4*)(xr + 32 * hb + 4 * s4) : make_float4(0, 0, 0, 0);
        bq32[q][4 * s4 + 0] = raw.x;
        bq32[q][4 * s4 + 1] = raw.y;
        bq32[q][4 * s4 + 2] = raw.z;
        bq32[q][4 * s4 + 3] = raw.w;
        acc = fmaf(raw.x, raw.x, acc);
        acc = fmaf(raw.y, raw.y, acc);
        acc = fmaf(raw.z, raw.z, acc);
        acc = fmaf(raw.w, raw.w, acc);
      }
    }
    nrm2[q] = acc + __shfl_xor(acc, 32);
  }
  if (token_scales != nullptr && wave_valid)  // lanes 0-31: group 0, lanes 32-63: group 1
    token_scales[(size_t)bh * L + tok_base + 32 * hb + n] = token_scale(hb ? nrm2[1] : nrm2[0]);
  // |x| rounded up, for the certification bound of every round
  const float xnorm[2] = {sqrtf(nrm2[0]) * 1.000001f, sqrtf(nrm2[1]) * 1.000001f};

  // Largest column norm of each round, from the per-block bounds, into LDS once,
  // so that a round end reads it without a load and a reduction (NaN bounds are
  // skipped, as fmaxf would).
  if (threadIdx.x < kMaxHashes) sRho[threadIdx.x] = 0u;
  __syncthreads();
  {
    const int nblk = (halfp + 63) / 64;
    for (int i = (int)threadIdx.x; i < n_h * nblk; i += 256) {
      const float v = colmax[i];
      if (v == v) atomicMax(&sRho[i / nblk], __float_as_uint(v));
    }
  }

  // Rotation blocks of CB columns, over all rounds in order.  halfp is a multiple
  // of CB and rot_t is [n_h][halfp][D], so block k is the k-th contiguous run of
  // CB rows.  bf16 moves a block with direct loads (dma, below).  fp32 moves it
  // through registers in parts of 64 columns: part q is the q-th contiguous run
  // of 64 rows (block q / kParts, LDS buffer (q / kParts) & 1), and thread t
  // moves its 16-byte pieces t + 256 i at fixed offsets.  While block k is
  // used, the parts of block k+1 are stored to the other buffer one after
  // another, each as soon as it is in registers, and the next part is loaded
  // in its place.
  constexpr int kPieces = BF16 ? 8 : 16;  // 16-byte pieces per 64-element row
  constexpr int kPer = BF16 ? 8 : 4;      // elements per piece
  constexpr int kPF = 64 * kPieces / 256;
  constexpr uint32_t kPartBytes = 64 * kD * sizeof(T);
  constexpr int kT = CB / 32;       // 32-column tiles per block
  constexpr int kParts = CB / 64;   // parts per block
  static_assert(CB % 64 == 0 && kT > kParts, "an even number of tiles, and a step before each part's store");
  const int nbpr = halfp / CB;  // blocks per round
  const int total = n_h * nbpr;
  const int tparts = total * kParts;
  int lds_off[kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    lds_off[i] = (c / kPieces) * kRow + (c % kPieces) * kPer;
  }
  const uint32_t piece_off = 16u * threadIdx.x;
  u32x4 pf[kPF];  // native vector type: HIP's uint4 struct copies defeat register promotion here
  auto prefetch = [&](int q) {
    const char* src = (const char*)rot_t + (size_t)q * kPartBytes;  // wave-uniform
#pragma unroll
    for (int i = 0; i < kPF; ++i) pf[i] = *(const u32x4*)(src + (piece_off + 4096u * i));
  };
  auto stage = [&](int q) {
    T* dst = (((q / kParts) & 1) ? sR1 : sR0) + (q % kParts) * 64 * kRow;
#pragma unroll
    for (int i = 0; i < kPF; ++i) *(u32x4*)(dst + lds_off[i]) = pf[i];
  };
  // bf16: block k goes straight from memory to dst (global_load_lds, no
  // registers).  Piece p of row r is stored at position p ^ (r & 7) ^ ((r >> 3) & 1):
  // the 16 rows an operand read covers at a time (rows r and r + 8 included)
  // then fall on distinct LDS banks.  One wave instruction fills 8 rows: lane
  // l writes the 16-byte slot l of them (row l / 8, position l % 8), so it
  // loads source piece (l % 8) ^ (l / 8) ^ (g & 1) of 8-row group g.  Wave w
  // fills the groups w, w + 4, ...
  auto dma = [&](T* dst, int k) {
    const char* src = (const char*)rot_t + (size_t)k * (CB * kD * sizeof(T));  // wave-uniform
#pragma unroll
    for (int i = 0; i < CB / 32; ++i) {
      const int g = wave + 4 * i;
      const uint32_t soff =
          128u * (uint32_t)(lane >> 3) + 16u * (uint32_t)((lane & 7) ^ (lane >> 3) ^ (g & 1));
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + 1024u * g + soff),
                                       (__attribute__((address_space(3))) void*)(dst + 8 * g * kRow), 16, 0, 0);
    }
  };

  // Software pipeline over the stream of 32-column tiles (kT per staged block):
  // the MFMAs of the next tile are issued between the top-2 selection steps of
  // the current one, so matrix and vector work of one wave overlap.  Blocks are
  // double-buffered in LDS (block k in sR0 for even k, sR1 for odd), one
  // barrier per block.
  uint32_t m1[2] = {0u, 0u}, m2[2] = {0u, 0u};  // running top-2 keys per token group
  // One pipeline step: the MFMAs of tile t_next (from LDS buffer buf) into
  // (n0, n1), interleaved in issue order with the top-2 selection of the
  // finished tile tg_cur in (c0, c1).  In-order issue means a dependent MFMA
  // blocks the instructions behind it, so each MFMA is followed by a share of
  // the selection (two pair-steps, ten VALU ops) and sched_barrier pins that
  // order.
  auto step = [&](const T* buf, int t_next, f32x16& n0, f32x16& n1, int tg_cur, const f32x16& c0,
                  const f32x16& c1) {
    const uint32_t cbase = lowmask - 16u * (uint32_t)tg_cur;
    auto pair = [&](int q, int e) {
      const f32x16& c = q ? c1 : c0;
      const uint32_t a = (__float_as_uint(c[e]) & kmask_v) | (cbase - e);
      const uint32_t b = (__float_as_uint(c[e + 1]) & kmask_v) | (cbase - e - 1);
      const uint32_t hi = umax3(m1[q], a, b);
      m2[q] = max(m2[q], umed3(m1[q], a, b));
      m1[q] = hi;
    };
    n0 = f32x16{};
    n1 = f32x16{};
    const T* arow = buf + (32 * t_next + n) * kRow;
    if constexpr (BF16) {
      bf16x8 a[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = *(const bf16x8*)(arow + 8 * ((2 * s + hb) ^ (n & 7) ^ ((n >> 3) & 1)));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], bq16[0][s], n0, 0, 0, 0);
        pair(0, 4 * s);
        pair(0, 4 * s + 2);
        __builtin_amdgcn_sched_barrier(0);
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], bq16[1][s], n1, 0, 0, 0);
        pair(1, 4 * s);
        pair(1, 4 * s + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // fp32: 64 MFMA 32x32x2 per tile, one pair-step after every fourth.
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4) {
        float4 a4 = *(const float4*)(arow + 32 * hb + 4 * s4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          n0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bq32[0][4 * s4 + e], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bq32[1][4 * s4 + e], n1, 0, 0, 0);
        }
        pair(0, 2 * s4);
        pair(1, 2 * s4);
      }
    }
  };
  // First tile of the stream: MFMAs only.
  auto project0 = [&](f32x16& n0, f32x16& n1) {
    n0 = f32x16{};
    n1 = f32x16{};
    const T* arow = sR0 + n * kRow;
    if constexpr (BF16) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = *(const bf16x8*)(arow + 8 * ((2 * s + hb) ^ (n & 7) ^ ((n >> 3) & 1)));
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq16[0][s], n0, 0, 0, 0);
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq16[1][s], n1, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4) {
        const float4 a4 = *(const float4*)(arow + 32 * hb + 4 * s4);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          n0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bq32[0][4 * s4 + e], n0, 0, 0, 0);
          n1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bq32[1][4 * s4 + e], n1, 0, 0, 0);
        }
      }
    }
  };
  f32x16 ea0, ea1, ob0, ob1;  // accumulators of the even / odd tile of a block
  if constexpr (BF16) {
    dma(sR0, 0);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
  } else {
#pragma unroll
    for (int h = 0; h < kParts; ++h) {
      prefetch(h);
      stage(h);
    }
    if (tparts > kParts) prefetch(kParts);
  }
  __syncthreads();
  project0(ea0, ea1);
  int r = 0, cb = 0;  // round and first column of block it
  // One block: cur holds block it, nxt receives block it+1 (the other buffer,
  // last read before the previous block's barrier).
  auto block = [&](const T* cur, T* nxt, int it) {
    // bf16: block it+1 is loaded straight into nxt while block it is used.
    if constexpr (BF16)
      if (it + 1 < total) dma(nxt, it + 1);
    // Tiles 1 .. kT-1 of block it (MFMAs of tile t, selection of tile t - 1),
    // alternating between the two accumulator pairs.  fp32: after step
    // t <= kParts, part t - 1 of block it+1 (in registers since the previous
    // store) goes to nxt and the next part is loaded.
#pragma unroll
    for (int t = 1; t < kT; ++t) {
      if (t & 1)
        step(cur, t, ob0, ob1, (cb >> 5) + t - 1, ea0, ea1);
      else
        step(cur, t, ea0, ea1, (cb >> 5) + t - 1, ob0, ob1);
      if constexpr (!BF16) {
        const int q = (it + 1) * kParts + t - 1;
        if (t <= kParts && q < tparts) {
          stage(q);
          if (q + 1 < tparts) prefetch(q + 1);
        }
      }
    }
    if constexpr (BF16) __builtin_amdgcn_s_waitcnt(0);  // this wave's part of block it+1 has landed
    __syncthreads();
    // After the last block this reads the other (stale but in-bounds) buffer
    // and the result is unused: it keeps the step free of branches.
    step(nxt, 0, ea0, ea1, (cb >> 5) + kT - 1, ob0, ob1);
    cb += CB;
    if (cb < halfp) return;
    cb = 0;

    // End of round r: merge with the partner lane (same tokens, the other 16 rows
    // of each tile), decode the winner, certify, take the sign.
    // largest column norm of this round's rotation
    const float eps_scale = 65.0f * 0x1p-23f * __uint_as_float(sRho[r]);
    int jstar[2];
    bool certified[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      // lanes l and l + 32 hold the same tokens: both see (lower lane's, upper
      // lane's) key through one swap of the wave's halves
      const auto k1 = __builtin_amdgcn_permlane32_swap(m1[q], m1[q], false, false);
      const auto k2 = __builtin_amdgcn_permlane32_swap(m2[q], m2[q], false, false);
      const uint32_t M1 = max(k1[0], k1[1]);
      const uint32_t M2 = max(min(k1[0], k1[1]), max(k2[0], k2[1]));
      // Half of the tile the winner's row lies in (ties of identical keys are
      // equal-value ties, which are never certified, so any choice works).
      const int win_h = k1[0] < k1[1] ? 1 : 0;
      const uint32_t u = lowmask - (M1 & lowmask);  // 16 tg + e
      const int tg = (int)(u >> 4), e = (int)(u & 15);
      jstar[q] = 32 * tg + 8 * (e >> 2) + 4 * win_h + (e & 3);
      const float t1 = __uint_as_float(M1 & kmask), t2 = __uint_as_float(M2 & kmask);
      const float eps = eps_scale * xnorm[q];
      const int ebits = (int)((M1 >> 23) & 0xFFu) - 23 + ibits;
      const float delta = ebits >= 1 ? __uint_as_float((uint32_t)ebits << 23) : 0x1p-126f;
      certified[q] = (t1 - t2) > 2.0f * eps + delta;
    }
    // Sign of each winner: its score recomputed from this lane's half of the
    // token (the MFMA operand registers) and the partner lane's half.  When the
    // decision is certified |score| > 2 eps, so the fp32 sign is exact.  The
    // rotation rows of both groups are loaded before either is used, so the
    // round end waits for one round trip to memory, not one per load.
    int32_t result[2];
    if constexpr (BF16) {
      u32x4 w[2][4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const T* rr = rot_t + ((size_t)r * halfp + jstar[q]) * kD + 8 * hb;
#pragma unroll
        for (int s = 0; s < 4; ++s) w[q][s] = *(const u32x4*)(rr + 16 * s);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        // v_dot2c_f32_bf16: two exact bf16 products added to the fp32 sum with one
        // rounding per step (measured), within the same error bound as the MFMA sum.
        float dp = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 xb = __builtin_bit_cast(u32x4, bq16[q][s]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // (elements copied to scalars first: a bit_cast applied directly to a
            // vector element is lowered as element 0 by this compiler)
            const uint32_t wk = w[q][s][k], xk = xb[k];
            dp = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wk), __builtin_bit_cast(bf16x2, xk),
                                                 dp, false);
          }
        }
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(dp), __float_as_uint(dp), false, false);
        dp = __uint_as_float(h[0]) + __uint_as_float(h[1]);
        result[q] = dp > 0.f ? jstar[q] : jstar[q] + half;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const T* rr = rot_t + ((size_t)r * halfp + jstar[q]) * kD;
        float dp = 0.f;
#pragma unroll
        for (int s4 = 0; s4 < 8; ++s4) {
          const float4 a4 = *(const float4*)(rr + 32 * hb + 4 * s4);
          dp = fmaf(a4.x, bq32[q][4 * s4 + 0], dp);
          dp = fmaf(a4.y, bq32[q][4 * s4 + 1], dp);
          dp = fmaf(a4.z, bq32[q][4 * s4 + 2], dp);
          dp = fmaf(a4.w, bq32[q][4 * s4 + 3], dp);
        }
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(dp), __float_as_uint(dp), false, false);
        dp = __uint_as_float(h[0]) + __uint_as_float(h[1]);
        result[q] = dp > 0.f ? jstar[q] : jstar[q] + half;
      }
    }
    if (wave_valid) {
      // Lanes 0-31 store group 0, lanes 32-63 group 1: 64 consecutive tokens.
      const int tok = tok_base + 32 * hb + n;
      const size_t idx = ((size_t)bh * n_h + r) * L + tok;
      const bool cert = hb ? certified[1] : certified[0];
      if (cert) {
        buckets[idx] = hb ? result[1] : result[0];
      } else {
        buckets[idx] = -1;
        const int slot = atomicAdd(fix_count, 1);
        fix_queue[slot] = (int)idx;
      }
    }
    m1[0] = m1[1] = m2[0] = m2[1] = 0u;
    ++r;
  };
  if constexpr (BF16) {
    // unrolled by two, so that each call's buffers are fixed arrays
    for (int it = 0; it < total; it += 2) {
      block(sR0, sR1, it);
      if (it + 1 < total) block(sR1, sR0, it + 1);
    }
  } else {
    for (int it = 0; it < total; ++it) block((it & 1) ? sR1 : sR0, (it & 1) ? sR0 : sR1, it);
  }
}


// ---------------------------------------------------------------------------
// Float64 re-decision of queued tokens, one wave per token-round (grid-stride
// over the queue), in two phases.
//  1. fp32 scores of every column, within the certification's eps of the exact
//     ones.  The wave reads the round's transposed rotation front to back with
//     each load instruction covering whole rows: lane l holds 16-byte piece
//     l % P of row (64 / P) i + l / P (P pieces per row), so an instruction
//     touches 64 / P cache lines, not 64 as a column per lane would.  A batch of
//     P instructions covers 64 rows; DPP adds over the P lanes of a row finish
//     the sums, and lane l keeps row (64 / P)(l % P) + l / P of the batch.
//  2. The exact argmax lies among the columns whose fp32 score is within 2 eps
//     (plus a denormal allowance) of the best one: each is scored as a float64
//     sum of exact products by the whole wave (lane d holds element d), lowest
//     index on equal values.  More candidates than kMaxCand (tied or
//     degenerate inputs): every column in float64, lane-parallel.
// ---------------------------------------------------------------------------
constexpr int kMaxCand = 8;
constexpr int kFixWaves = 4;
constexpr int kMaxHalfp = 2048;
static_assert(kMaxHalfp >= kMaxBuckets / 2 && kMaxHalfp % 64 == 0, "score slots for the largest n_b");

// A lane's value moved by a DPP lane pattern (CTRL: the gfx9 dpp_ctrl code).
template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// fp32 dot product of one 16-byte piece of x and of a rotation row.
__device__ inline float piece_dot(const uint4& a, const uint4& b, uint16_t) {
  const uint32_t xa[4] = {a.x, a.y, a.z, a.w}, ra[4] = {b.x, b.y, b.z, b.w};
  float acc = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t xw = xa[h], rw = ra[h];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xw), __builtin_bit_cast(bf16x2, rw), acc, false);
  }
  return acc;
}
__device__ inline float piece_dot(const uint4& a, const uint4& b, float) {
  float acc = __uint_as_float(a.x) * __uint_as_float(b.x);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
}

template <typename T>
__global__ __launch_bounds__(kFixWaves * 64) void fixup_kernel(const T* __restrict__ qk,
                                                               const T* __restrict__ rot_t,
                                                               const float* __restrict__ colmax,
                                                               int32_t* __restrict__ buckets,
                                                               const int* __restrict__ fix_queue,
                                                               const int* __restrict__ fix_count, int L, int n_h,
                                                               int half, int halfp) {
  constexpr int P = kD * (int)sizeof(T) / 16;  // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) float ssc[kFixWaves][kMaxHalfp];  // |fp32 score|, slot 64 g + lane of batch g
  const int lane = threadIdx.x & 63;
  float* sc = ssc[threadIdx.x >> 6];
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  const int count = *fix_count;
  const int nbatch = halfp >> 6;  // also the 64-column blocks of colmax
  for (int it = gw; it < count; it += nw) {
    const int idx = fix_queue[it];
    const int tok = idx % L;
    const int br = idx / L;
    const int r = br % n_h;
    const int bh = br / n_h;
    const T* x = qk + ((size_t)bh * L + tok) * kD;
    const uint4 xp = ((const uint4*)x)[lane % P];
    const double xd = to_f64(x[lane]);
    const uint4* R4 = (const uint4*)(rot_t + (size_t)r * halfp * kD);
    // largest column norm of the round (rounded up): one block bound per lane
    // (nbatch <= 32), then a wave maximum
    float rho = lane < nbatch ? colmax[r * nbatch + lane] : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rho = fmaxf(rho, __shfl_xor(rho, off));
    // Phase 1.
    float m = 0.f;
    for (int g = 0; g < nbatch; ++g) {
      uint4 rw[P];
#pragma unroll
      for (int i = 0; i < P; ++i) rw[i] = R4[(size_t)64 * (P * g + i) + lane];
      float V[P];
#pragma unroll
      for (int i = 0; i < P; ++i) V[i] = piece_dot(xp, rw[i], T());
      // Sum each row over the P lanes that hold its pieces (a group of P
      // consecutive lanes) with DPP moves inside the group: swap neighbours,
      // swap pairs, mirror the 8 lanes, (P = 16) mirror the 16.  Every lane ends
      // with the same sums (each step adds two equal-shaped partial sums, and
      // fp32 addition is commutative); lane l keeps the one of row
      // (64 / P)(l % P) + l / P.
#pragma unroll
      for (int i = 0; i < P; ++i) {
        V[i] += dpp_f32<0xB1>(V[i]);   // quad_perm [1, 0, 3, 2]: lane ^ 1
        V[i] += dpp_f32<0x4E>(V[i]);   // quad_perm [2, 3, 0, 1]: lane ^ 2
        V[i] += dpp_f32<0x141>(V[i]);  // row_half_mirror: lane i <-> 7 - i
        if constexpr (P == 16) V[i] += dpp_f32<0x140>(V[i]);  // row_mirror: i <-> 15 - i
      }
      float own = V[0];
#pragma unroll
      for (int i = 1; i < P; ++i) own = (lane & (P - 1)) == i ? V[i] : own;
      const int row = 64 * g + (64 / P) * (lane % P) + lane / P;
      const float a = fabsf(own);
      sc[64 * g + lane] = row < half ? a : -INFINITY;
      m = row < half ? fmaxf(m, a) : m;
    }
    float n2 = piece_dot(xp, xp, T());
#pragma unroll
    for (int h = 1; h < P; h <<= 1) n2 += __shfl_xor(n2, h);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    // Each fp32 score passes through at most 8 roundings (4 in the piece, up to
    // 4 in the reduction): far inside eps.  A flushed denormal product errs by at
    // most 2^-126, 64 of them by 2^-120, for each of the two scores compared.
    const float eps = 65.0f * 0x1p-23f * rho * (sqrtf(n2) * 1.00001f);
    const double thr64 = (double)m - (2.0 * (double)eps + 0x1p-118);
    float thr = (float)thr64;
    if ((double)thr > thr64) thr = nextafterf(thr, -INFINITY);
    uint32_t mask = 0;  // bit g: this lane's row of batch g is a candidate
    for (int g = 0; g < nbatch; ++g) mask |= (sc[64 * g + lane] >= thr ? 1u : 0u) << g;
    // Phase 2.
    int cj[kMaxCand];
    int ncand = 0;  // candidates found (the first ncand entries of cj; wave-uniform)
#pragma unroll
    for (int c = 0; c < kMaxCand; ++c) {
      const uint64_t bal = __ballot(mask != 0);
      if (bal == 0) {
        cj[c] = -1;
        continue;
      }
      ++ncand;
      const int src = __builtin_ctzll(bal);
      const uint32_t ms = __shfl(mask, src);
      cj[c] = 64 * __builtin_ctz(ms) + (64 / P) * (src % P) + src / P;
      if (lane == src) mask &= mask - 1u;
    }
    const bool overflow = __ballot(mask != 0) != 0;
    // Each candidate's float64 sum is certified against its rounding: the exact
    // sum S and the computed one differ by at most err * sum|x_d r_d| (err =
    // 8 * 2^-53 for the 6-level butterfly below, 72 * 2^-53 for a serial fma
    // chain of 64 terms; sum|x_d r_d| itself computed the same way).  The winner
    // is decided in float64 when its interval lies strictly above every other
    // candidate's and away from zero (so its sign, which picks column j or
    // j + half, is exact); otherwise every candidate that may win is compared
    // exactly (exact_abs_compare), lowest index on equal values.
    constexpr double kErrTree = 0x1p-50, kErrSerial = 72.0 * 0x1p-53;
    double* ex = (double*)sc;  // the wave's LDS area, free after phase 1: 1024 doubles
    double* pa = ex;           // products of the current best column
    double* pb = ex + 64;      // products of the column it is compared with
    double* e1 = ex + 128;     // expansions: 64 + 64 + 128
    double* e2 = ex + 192;
    double* e3 = ex + 256;
    const T* rrow = rot_t + (size_t)r * halfp * kD;  // this round's transposed rotation
    int best_i = 0x7FFFFFFF;
    int best_j = -1;            // column of a float64 winner that could not be certified
    uint32_t cmask = 0;         // this lane's columns j = lane + 64 k that may beat it (bit k)
    uint32_t cand8 = 0;         // or: candidates c of the short list that may (bit c)
    if (!overflow) {
      T rv[kMaxCand];
#pragma unroll
      for (int c = 0; c < kMaxCand; ++c) rv[c] = cj[c] >= 0 ? rrow[(size_t)cj[c] * kD + lane] : T(0);
      double S[kMaxCand], A[kMaxCand];
      const int nc = __builtin_amdgcn_readfirstlane(ncand);
#pragma unroll
      for (int c = 0; c < kMaxCand; ++c) {
        S[c] = A[c] = 0.0;
        if (c >= nc) continue;  // empty slots skip the two float64 butterflies
        double p = xd * to_f64(rv[c]), q = fabs(p);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          p += __shfl_xor(p, off);
          q += __shfl_xor(q, off);
        }
        S[c] = p;
        A[c] = q;
      }
      int bc = 0;
      double bv = -1.0;
#pragma unroll
      for (int c = 0; c < kMaxCand; ++c) {
        if (cj[c] < 0) break;
        const double v = fabs(S[c]);
        const int i = S[c] < 0.0 ? cj[c] + half : cj[c];  // the larger of +p (index j) and -p (index j + half)
        if (v > bv || (v == bv && i < best_i)) {
          bv = v;
          best_i = i;
          bc = c;
        }
      }
      const double eb = kErrTree * A[bc];
      bool ok = bv > eb || A[bc] == 0.0;
#pragma unroll
      for (int c = 0; c < kMaxCand; ++c)
        if (cj[c] >= 0 && c != bc && !(bv - eb > fabs(S[c]) + kErrTree * A[c])) {
          ok = false;
          cand8 |= 1u << c;
        }
      if (!ok) {
        best_j = cj[bc];
        best_i = 0x7FFFFFFF;
      }
    } else {
      // Every column in float64, lane-parallel (x re-read from memory, cached, to
      // keep this rare path's registers low).
      double bv = -1.0, be = 0.0;
      int bj = -1;
      for (int j = lane; j < half; j += 64) {
        const T* rr = rrow + (size_t)j * kD;
        double p = 0.0, q = 0.0;
        for (int d = 0; d < kD; ++d) {
          const double t = to_f64(x[d]) * to_f64(rr[d]);
          p += t;
          q += fabs(t);
        }
        const double v = fabs(p);
        const int i = p < 0.0 ? j + half : j;
        if (v > bv || (v == bv && i < best_i)) {
          bv = v;
          best_i = i;
          bj = j;
          be = kErrSerial * q;
        }
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off), oe = __shfl_xor(be, off);
        const int oi = __shfl_xor(best_i, off), oj = __shfl_xor(bj, off);
        if (ov > bv || (ov == bv && oi < best_i)) {
          bv = ov;
          best_i = oi;
          bj = oj;
          be = oe;
        }
      }
      // Columns whose interval reaches the winner's.
      for (int j = lane, k = 0; j < half; j += 64, ++k) {
        if (j == bj) continue;
        const T* rr = rrow + (size_t)j * kD;
        double p = 0.0, q = 0.0;
        for (int d = 0; d < kD; ++d) {
          const double t = to_f64(x[d]) * to_f64(rr[d]);
          p += t;
          q += fabs(t);
        }
        if (!(bv - be > fabs(p) + kErrSerial * q)) cmask |= 1u << k;
      }
      const bool sign_ok = bv > be || be == 0.0;
      if (!sign_ok || __ballot(cmask != 0) != 0) {
        best_j = bj;
        best_i = 0x7FFFFFFF;
      }
    }
    if (best_j >= 0) {
      // Exact decision among the winner and the columns that may beat it.  Lane d
      // writes product d; lane 0 runs the expansions.  (One wave's LDS
      // operations execute in order, so lane 0 reads what every lane wrote.)
      pa[lane] = xd * to_f64(rrow[(size_t)best_j * kD + lane]);
      __builtin_amdgcn_wave_barrier();
      int sbest = 2;  // sign of the best column's sum once known
      auto challenge = [&](int j) {
        const T rj = rrow[(size_t)j * kD + lane], rb = rrow[(size_t)best_j * kD + lane];
        if (__ballot(rj != rb) == 0ull) {
          // identical columns: equal sums and signs, so the lower column wins
          if (j < best_j) best_j = j;
          return;
        }
        pb[lane] = xd * to_f64(rj);
        __builtin_amdgcn_wave_barrier();
        int cmp = 0, sa = 0, sbj = 0;
        if (lane == 0) cmp = exact_abs_compare(pa, pb, kD, e1, e2, e3, sa, sbj);
        cmp = __shfl(cmp, 0);
        sa = __shfl(sa, 0);
        sbj = __shfl(sbj, 0);
        const int ia = sa < 0 ? best_j + half : best_j, ib = sbj < 0 ? j + half : j;
        if (cmp < 0 || (cmp == 0 && ib < ia)) {
          best_j = j;
          sbest = sbj;
          pa[lane] = pb[lane];
          __builtin_amdgcn_wave_barrier();
        } else {
          sbest = sa;
        }
      };
      if (!overflow) {
#pragma unroll
        for (int c = 0; c < kMaxCand; ++c)
          if (cand8 & (1u << c)) challenge(cj[c]);
      } else {
        for (uint64_t bal = __ballot(cmask != 0); bal != 0ull; bal = __ballot(cmask != 0)) {
          const int src = __builtin_ctzll(bal);
          const int k = __builtin_ctz(__shfl(cmask, src));
          if (lane == src) cmask &= cmask - 1u;
          challenge(src + 64 * k);
        }
      }
      if (sbest == 2) {
        // no exact comparison was made (identical columns, or only the winner's
        // sign was uncertain): the sign of its sum, exactly
        int sg = 0;
        if (lane == 0) {
          int n = 0;
          for (int k = 0; k < kD; ++k) n = grow_expansion(e1, n, pa[k]);
          sg = expansion_sign(e1, n);
        }
        sbest = __shfl(sg, 0);
      }
      best_i = sbest < 0 ? best_j + half : best_j;
    }
    // With finite inputs the best fp32 score is always a candidate; non-finite
    // ones leave the first pass's decision in place.
    if (lane == 0 && best_i != 0x7FFFFFFF) buckets[idx] = best_i;
  }
}

__global__ void fill_zero_kernel(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

hipError_t launch_prep(const void* rot, void* rot_t, float* colmax, int* fix_count, int n_h, int n_b,
                       lsh_dtype dt, hipStream_t s) {
  const int half = n_b / 2, halfp = padded_half(n_b), nblk = (halfp + 63) / 64;
  if (dt == LSH_BF16)
    prep_kernel<uint16_t><<<n_h * nblk, 256, 0, s>>>((const uint16_t*)rot, (uint16_t*)rot_t, colmax, fix_count,
                                                     half, halfp, nblk);
  else
    prep_kernel<float><<<n_h * nblk, 256, 0, s>>>((const float*)rot, (float*)rot_t, colmax, fix_count, half,
                                                  halfp, nblk);
  return hipGetLastError();
}

hipError_t launch_hash(const void* qk, const void* rot_t, const float* colmax, int32_t* buckets,
                       int* fix_queue, int* fix_count, float2* token_scales, int BH, int L, int n_b, int n_h,
                       lsh_dtype dt, hipStream_t s) {
  const int half = n_b / 2, halfp = padded_half(n_b);
  // Codes 16 tg + e < halfp / 2 must fit in the low bits of the key.
  int ibits = 0;
  while ((1 << ibits) < halfp / 2) ++ibits;
  const uint32_t lowmask = (1u << ibits) - 1u;
  const unsigned grid = (unsigned)((L + kHashTok - 1) / kHashTok) * (unsigned)BH;
  // bf16: 128-column passes (half the barriers) when the padded rotation splits
  // into them, else 64.
  if (dt == LSH_BF16 && halfp % 128 == 0)
    hash_kernel<true, 128><<<grid, 256, 0, s>>>((const uint16_t*)qk, (const uint16_t*)rot_t, colmax, buckets,
                                                fix_queue, fix_count, token_scales, L, n_h, half, halfp, lowmask,
                                                ibits);
  else if (dt == LSH_BF16)
    hash_kernel<true, 64><<<grid, 256, 0, s>>>((const uint16_t*)qk, (const uint16_t*)rot_t, colmax, buckets, fix_queue,
                                           fix_count, token_scales, L, n_h, half, halfp, lowmask, ibits);
  else
    hash_kernel<false, 64><<<grid, 256, 0, s>>>((const float*)qk, (const float*)rot_t, colmax, buckets, fix_queue,
                                            fix_count, token_scales, L, n_h, half, halfp, lowmask, ibits);
  return hipGetLastError();
}

hipError_t launch_fixup(const void* qk, const void* rot_t, const float* colmax, int32_t* buckets,
                        const int* fix_queue, const int* fix_count, int L, int n_b, int n_h, lsh_dtype dt,
                        hipStream_t s) {
  const int half = n_b / 2, halfp = padded_half(n_b);
  if (halfp > kMaxHalfp) return hipErrorInvalidValue;
  if (dt == LSH_BF16)
    fixup_kernel<uint16_t><<<1024, kFixWaves * 64, 0, s>>>((const uint16_t*)qk, (const uint16_t*)rot_t, colmax,
                                                          buckets, fix_queue, fix_count, L, n_h, half, halfp);
  else
    fixup_kernel<float><<<1024, kFixWaves * 64, 0, s>>>((const float*)qk, (const float*)rot_t, colmax, buckets,
                                                       fix_queue, fix_count, L, n_h, half, halfp);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, size_t n, hipStream_t s) {
  fill_zero_kernel<<<1024, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace lsh
