// Backward of the shared-QK LSH attention forward pass: gradients with respect
// to the shared query/key vectors and the values.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer): tokens are hashed,
// sorted by bucket and attended in equal chunks (each chunk and the one before
// it), and several rounds are unioned.  Hashing and sorting are piecewise
// constant, so the forward's permutation is reused and the gradient flows
// through the chunk attention and the combine only.
//
// Maths.  For query slot g of token i in round r and key occurrence k (token j)
// in its window, with P_gk the round's softmax weight and w_g = exp(lse_r(i) -
// LSE_i) the combine weight, the loss sum_i dout_i . out_i + dLSE_i LSE_i gives
//   dlogit_gk = w_g P_gk (dout_i . v_j + c_i),   c_i = dLSE_i - dout_i . out_i
//   dv_j     += w_g P_gk dout_i
// (the per-round output o_r cancels out of the combine's derivative).  With
// logit = x_i . khat_j / 8, khat_j = x_j / max(|x_j|, 1e-12) and kn_j = 1 /
// (8 max(|x_j|, 1e-12)):
//   dx_i (query role) += dlogit_gk kn_j x_j
//   a_j              += dlogit_gk x_i,     dx_j (key role) = kn_j (a_j - khat_j (khat_j . a_j))
// (kn_j a_j when |x_j| <= 1e-12).  The self logit is the constant -1e5 and a
// causally dropped key has weight 0: neither passes a gradient to x.
//
// Kernels:
//   bwd_prep   - per token: the combine weights w of its n_h rounds with w c_i
//                (token-major, one coalesced record per token), its key scales.
//   attn_bwd   - per block, 8 consecutive chunks as keys.  Step c takes the
//                queries of chunk c against the keys of chunks c-1 and c (the
//                forward's window).  A chunk's keys are attended by the
//                queries of its own chunk and of the next one, so the two
//                waves that own a ring slot's keys keep that chunk's dv, a and
//                dq accumulators over two consecutive steps and then write the
//                slot's finished dx (query role + key role) and dv.  One extra
//                step at the end of the run completes its last chunk; the
//                first step's look-back keys belong to the previous run and
//                only feed the dq of the first chunk.  No atomics: every slot
//                is finished inside one block.
//   bwd_reduce - per token: dx_i = sum over its n_h slots, dv_i likewise.
//
// gfx950 layout of attn_bwd (8 waves; wave w owns keys 16 (w & 3) .. +15 of
// ring slot w >> 2):
//   S = Q K^T and dP = dO V^T on MFMA with queries as rows, so each lane holds
//   4 consecutive queries of one key;  dV^T += dO^T Pw and A^T += Xq^T dS take
//   the lane's own Pw / dS as the B operand, the A operand straight from the
//   LDS row copies of dO and x through the gfx950 transposing LDS read
//   (ds_read_b64_tr_b16, tr_operand), with the queries in the order of the B
//   operand; dS kn is written to LDS (bf16) and the key-owning waves of the
//   current chunk form dQ^T = Xk^T (dS kn)^T over all 128 keys for their 16
//   queries, whose layout equals their own key accumulators.  The dS tile
//   reuses the dO row buffer (a barrier separates the uses).  The transposed
//   operands put dims 8g + 4h + e (h = 0, 1) of each 32-dim half in the rows
//   of lane group g, so each lane's finished dx and dv are two contiguous
//   16-byte pieces.  The bf16 tiles use unpadded rows with XOR-swizzled 16-byte
//   pieces (xoff / voff).  fp32 inputs take the fp32 MFMA and read the
//   operands element by element from the row copies.
#include "lsh_bwd.h"

namespace lsh {

namespace {

constexpr int kBwdChunksPerBlock = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSelf2 = -1.0e5f * kLog2e;
// A row whose lse is below this (natural log) has only its self key left: every
// real logit is at least -|x_i| / 8, far above the -1e5 of the self key.  The
// self key occurs once or twice in a window (its own chunk, and the look-back
// chunk when that belongs to the previous round), so a self-only row has lse
// -1e5 or -1e5 + ln 2 and each self copy the weight 1 or 1/2, told apart by
// the second threshold (both far from fp32 rounding at 1e5).
constexpr float kSelfOnlyLse = -1.0e5f + 1.0f;
constexpr float kSelfOnly2 = kSelfOnlyLse * kLog2e;
constexpr float kSelfTwice2 = (-1.0e5f + 0.35f) * kLog2e;

template <bool BF16>
struct BwdTraits;
template <>
struct BwdTraits<true> {
  using T = uint16_t;
  static constexpr int kXRow = 64;    // row copies: 64 dims (pieces swizzled, xoff)
  static constexpr int kSRow = 128;   // dS kn: 2 slots x 64 keys (voff)
};
template <>
struct BwdTraits<false> {
  using T = float;
  static constexpr int kXRow = 68;
  static constexpr int kSRow = 132;
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// bf16 LDS tiles keep rows unpadded and store 16-byte piece q of row r at
// piece q ^ (r mod pieces-per-row): the MFMA operand reads (16 lanes on 16
// rows, the 4 lane groups on 4 pieces) and the staging writes then run at the
// full LDS rate on gfx950 (padded 144- or 272-byte rows measured 1.6x slower
// for those reads).  Element offsets for 128-byte and 256-byte rows:
__device__ inline int xoff(int row, int piece) { return row * 64 + 8 * (piece ^ (row & 7)); }
__device__ inline int voff(int row, int piece) { return row * 128 + 8 * (piece ^ (row & 15)); }

// Column of chunk row r in the transposed operand layout: column 32h + 8g + 4b + e
// holds row 32h + 16b + 4g + e.
__device__ inline int permcol(int r) {
  return (r & ~31) | (((r >> 2) & 3) << 3) | (((r >> 4) & 1) << 2) | (r & 3);
}

// The value of the lane with index (this lane xor 1), resp. xor 2, within its
// quad of lanes (DPP quad permutations [1, 0, 3, 2] and [2, 3, 0, 1]).
__device__ inline uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ inline uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// A operand (16 dims x 32 rows of a bf16 row tile) of v_mfma_f32_16x16x32_bf16,
// read transposed from the row-major tile by ds_read_b64_tr_b16.  Within each
// 16-lane group, that instruction hands lane i element j of the 8-byte read of
// lane 4j + (i >> 2), element i & 3 (checked on the device).  Here lane
// 16g + 4j + r of the group reads row r0 + 4g + j (and r0 + 16 + 4g + j) at dims
// D(r) .. D(r) + 3, D(r) = 32 (dt >> 1) + 8r + 4 (dt & 1), so operand row i holds
// dim 32 (dt >> 1) + 8 (i >> 2) + 4 (dt & 1) + (i & 3) and lane group g the K
// indices 8g + b * 4 + e <-> tile rows r0 + 16b + 4g + e: the order of the
// lane's own probabilities as the B operand (permcol).
__device__ inline bf16x8 tr_operand(const uint16_t* tile, int r0, int dt, int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, r = lane & 3;
  const int piece = 4 * (dt >> 1) + r, sub = 4 * (dt & 1);
  const int ra = r0 + 4 * g + j;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + xoff(ra, piece) + sub));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + xoff(ra + 16, piece) + sub));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// bwd_prep: 16 lanes per token, 4 dims each.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ x_v, const void* __restrict__ out_v,
                                                       const void* __restrict__ dout_v,
                                                       const float* __restrict__ dlse,
                                                       const float* __restrict__ lse_sorted,
                                                       const int32_t* __restrict__ undo_idx,
                                                       float2* __restrict__ tok_w, float2* __restrict__ tok_scale,
                                                       int L, int n_h, size_t n_tokens) {
  const size_t t = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (t >= n_tokens) return;  // whole 16-lane groups leave together
  const size_t bh = t / L;
  const int i = (int)(t % L);
  const size_t n_slots = (size_t)n_h * L;
  float xs[4], os[4], ds[4];
  if constexpr (BF16) {
    const uint2 a = *(const uint2*)((const uint16_t*)x_v + t * kD + 4 * sub);
    const uint2 b = *(const uint2*)((const uint16_t*)out_v + t * kD + 4 * sub);
    const uint2 c = *(const uint2*)((const uint16_t*)dout_v + t * kD + 4 * sub);
    xs[0] = bf_lo(a.x); xs[1] = bf_hi(a.x); xs[2] = bf_lo(a.y); xs[3] = bf_hi(a.y);
    os[0] = bf_lo(b.x); os[1] = bf_hi(b.x); os[2] = bf_lo(b.y); os[3] = bf_hi(b.y);
    ds[0] = bf_lo(c.x); ds[1] = bf_hi(c.x); ds[2] = bf_lo(c.y); ds[3] = bf_hi(c.y);
  } else {
    const float4 a = *(const float4*)((const float*)x_v + t * kD + 4 * sub);
    const float4 b = *(const float4*)((const float*)out_v + t * kD + 4 * sub);
    const float4 c = *(const float4*)((const float*)dout_v + t * kD + 4 * sub);
    xs[0] = a.x; xs[1] = a.y; xs[2] = a.z; xs[3] = a.w;
    os[0] = b.x; os[1] = b.y; os[2] = b.z; os[3] = b.w;
    ds[0] = c.x; ds[1] = c.y; ds[2] = c.z; ds[3] = c.w;
  }
  float ss = 0.f, dd = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ss = fmaf(xs[e], xs[e], ss);
    dd = fmaf(ds[e], os[e], dd);
  }
  int g = 0;
  float l = -INFINITY;
  if (sub < n_h) {
    g = (int)min((uint32_t)undo_idx[(bh * n_h + sub) * L + i], (uint32_t)(n_slots - 1));
    l = lse_sorted[bh * n_slots + g];
  }
  float m = l;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    ss += __shfl_xor(ss, o);
    dd += __shfl_xor(dd, o);
    m = fmaxf(m, __shfl_xor(m, o));
  }
  const float e = sub < n_h ? __expf(l - m) : 0.f;
  float z = e;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o);
  const float c = (dlse == nullptr ? 0.f : dlse[t]) - dd;
  if (sub < n_h) {
    const float w = e * __builtin_amdgcn_rcpf(z);
    tok_w[t * n_h + sub] = make_float2(w, w * c);
  }
  if (sub == 0) {
    const float kn = 0.125f * __builtin_amdgcn_rcpf(fmaxf(__builtin_amdgcn_sqrtf(ss), 1e-12f));
    tok_scale[t] = make_float2(kLog2e * kn, kn);
  }
}

// ---------------------------------------------------------------------------
// attn_bwd
// ---------------------------------------------------------------------------
// NT: the per-slot dx and dv rows are written with non-temporal stores
// (stream_slot_rows: large, written once, read once by bwd_reduce).
template <bool BF16, bool CAUSAL, bool NT>
__global__ __launch_bounds__(512, 2) void attn_bwd_kernel(
    const typename BwdTraits<BF16>::T* __restrict__ qk, const typename BwdTraits<BF16>::T* __restrict__ v,
    const typename BwdTraits<BF16>::T* __restrict__ dout, const int32_t* __restrict__ sorted_idx,
    const float* __restrict__ lse_sorted, const float2* __restrict__ tok_w, const float2* __restrict__ tok_scale,
    typename BwdTraits<BF16>::T* __restrict__ dx_slot, typename BwdTraits<BF16>::T* __restrict__ dv_slot, int L,
    int n_h, int n_slots, int n_chunks, int blocks_per_bh) {
  using T = typename BwdTraits<BF16>::T;
  constexpr int kXRow = BwdTraits<BF16>::kXRow;
  constexpr int kSRow = BwdTraits<BF16>::kSRow;
  constexpr int kCPB = kBwdChunksPerBlock;
  constexpr int kLoads = BF16 ? 1 : 2;  // 16-byte row pieces per thread (8 per bf16 row, 16 per fp32 row)

  __shared__ __attribute__((aligned(16))) T sX[2][64 * kXRow];   // x rows per ring slot
  __shared__ __attribute__((aligned(16))) T sV[2][64 * kXRow];   // v rows per ring slot
  // dO rows; the bf16 dS kn tile reuses the space.
  constexpr int kDoElems = 64 * kXRow;
  constexpr int kSElems = 64 * kSRow;
  constexpr int kUnion = BF16 ? (kDoElems > kSElems ? kDoElems : kSElems) : kDoElems;
  __shared__ __attribute__((aligned(16))) T sDoBuf[kUnion];
  __shared__ __attribute__((aligned(16))) float sDsF[BF16 ? 1 : kSElems];  // fp32 dS kn tile
  __shared__ __attribute__((aligned(16))) float sKs2[2][64], sKn[2][64];   // key scales per slot
  __shared__ __attribute__((aligned(16))) float sLse2[64], sW[64], sWc[64];  // current queries
  __shared__ __attribute__((aligned(16))) int sPos[kCPB + 2][64];
  __shared__ int sSelfOnly;  // the current chunk has a self-only query row
  T* const sDO = sDoBuf;                      // [query][dim]
  uint16_t* const sDS16 = (uint16_t*)sDoBuf;  // [query][64 slot + permcol(key)] (bf16)

  const int bh = blockIdx.x / blocks_per_bh;
  const int c0 = (blockIdx.x % blocks_per_bh) * kCPB;
  const int c1 = min(n_chunks, c0 + kCPB);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sw = wave >> 2, kt = wave & 3;  // owned keys: rows 16 kt .. 16 kt + 15 of ring slot sw

  constexpr uint32_t kRowBytes = kD * sizeof(T);
  const char* xq = (const char*)(qk + (size_t)bh * L * kD);
  const char* vq = (const char*)(v + (size_t)bh * L * kD);
  const char* dq_in = (const char*)(dout + (size_t)bh * L * kD);
  const int32_t* sidx = sorted_idx + (size_t)bh * n_slots;
  const float* lseb = lse_sorted + (size_t)bh * n_slots;
  const float2* twb = tok_w + (size_t)bh * L * n_h;
  const int cpr = L / kChunk;  // chunks per round
  const float2* tsb = tok_scale + (size_t)bh * L;
  T* dxb = dx_slot + (size_t)bh * n_slots * kD;
  T* dvb = dv_slot + (size_t)bh * n_slots * kD;

  // Positions of steps c0-1 .. c1 (entry k <-> step c0-1+k, chunk (c0-1+k) mod n_chunks).
  for (int e = tid; e < (c1 - c0 + 2) * 64; e += 512) {
    const int k = e >> 6, r = e & 63;
    const int c = (c0 - 1 + k + n_chunks) % n_chunks;
    sPos[k][r] = (int)min((uint32_t)sidx[(size_t)c * kChunk + r], (uint32_t)(L - 1));
  }
  __syncthreads();

  // ---- gathers (registers) and commits (LDS) ----
  // rows: thread t holds 16-byte pieces (t & 7) * kLoads + i of row t >> 3.
  const int prow = tid >> 3, ppc = (tid & 7) * kLoads;
  uint4 xr[kLoads], vr[kLoads], dr[kLoads];
  float2 ksc = make_float2(0.f, 0.f), qsw = make_float2(0.f, 0.f);
  float qlse = 0.f;
  auto gather = [&](int k) {  // entry k: its keys, and (for every entry but the first) its queries
    const int* pos = sPos[k];
    const int chunk = (c0 - 1 + k + n_chunks) % n_chunks;
    const uint32_t off = (uint32_t)pos[prow] * kRowBytes + 16u * (uint32_t)ppc;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      xr[i] = *(const uint4*)(xq + off + 16u * i);
      vr[i] = *(const uint4*)(vq + off + 16u * i);
      dr[i] = *(const uint4*)(dq_in + off + 16u * i);
    }
    if (tid < 64) {
      ksc = tsb[pos[tid]];
      qlse = lseb[(size_t)chunk * kChunk + tid];
      qsw = twb[(size_t)pos[tid] * n_h + chunk / cpr];
    }
  };
  auto commit = [&](int slot, bool queries) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      if constexpr (BF16) {
        *(uint4*)(&sX[slot][xoff(prow, ppc)]) = xr[i];
        *(uint4*)(&sV[slot][xoff(prow, ppc)]) = vr[i];
      } else {
        *(uint4*)(&sX[slot][prow * kXRow + (ppc + i) * 4]) = xr[i];
        *(uint4*)(&sV[slot][prow * kXRow + (ppc + i) * 4]) = vr[i];
      }
    }
    if (tid < 64) {
      sKs2[slot][tid] = ksc.x;
      sKn[slot][tid] = ksc.y;
    }
    if (queries) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        if constexpr (BF16)
          *(uint4*)(&sDO[xoff(prow, ppc)]) = dr[i];
        else
          *(uint4*)(&sDO[prow * kXRow + (ppc + i) * 4]) = dr[i];
      }
      if (tid < 64) {
        sLse2[tid] = qlse * kLog2e;
        sW[tid] = qsw.x;
        sWc[tid] = qsw.y;
        const uint64_t so = __ballot(qlse < kSelfOnlyLse);  // wave 0: the chunk's 64 queries
        if (tid == 0) sSelfOnly = so != 0ull ? 1 : 0;
      }
    }
  };

  // prologue: step c0-1's keys (entry 0), then step c0's keys and queries (entry 1)
  gather(0);
  commit((c0 + 1) & 1, false);
  gather(1);
  commit(c0 & 1, true);
  __syncthreads();

  // accumulators of the owned keys: [dim tile], lane holds dims 16 dt + 4 grp + e of key kr
  f32x4 acc_v[4], acc_a[4], acc_q[4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      acc_v[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_a[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc_q[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  zero_acc();

  for (int c = c0; c <= c1; ++c) {
    // The lane's tile coordinates, re-derived each step from an opaque copy of the
    // lane id: the swizzled LDS addresses built from them are then computed inside
    // the step instead of being hoisted out of the loop, where they would hold
    // registers across it (the kernel is at the VGPR limit).
    int lane_v = lane;
    asm volatile("" : "+v"(lane_v));
    const int col = lane_v & 15, grp = lane_v >> 4;
    const int kr = 16 * kt + col;
    const int cur = c & 1, prv = cur ^ 1;
    const int ec = c - c0 + 1;  // sPos entry of step c
    if (c < c1) gather(ec + 1);  // next step's rows, in flight during this step
    const bool mine_cur = (sw == cur);
    const int ek = mine_cur ? ec : ec - 1;  // sPos entry of the owned keys
    const bool do_kv = mine_cur ? (c < c1) : (c > c0);
    const bool do_ds = (c < c1);
    const bool active = do_kv || do_ds;

    uint32_t dsk16[8];  // dS kn of the owned key for the 16 queries of this lane (bf16 pairs)
    float dskf[16];

    // Straight-line per chunk (no branch between query tiles, so the compiler can
    // overlap one tile's MFMAs with another's vector work); the look-back keys of
    // the run's first step are computed (their dS feeds dq) and then discarded.
    auto compute = [&](auto exact_tag) {
      constexpr bool EXACT = decltype(exact_tag)::value;
      const int kpos = sPos[ek][kr];
      const float ks2 = sKs2[sw][kr], kn = sKn[sw][kr];
      // Pw = w P (for dv) and dS (for x) from one query tile's S = Q K^T and dP = dO V^T
      // In a row with any real key the self key's weight exp(-1e5 - lse) is exactly 0,
      // so the self and causal masks are one compare that zeroes P.  Chunks with a
      // self-only row (lse near -1e5, flagged at commit) take the explicit path.
      auto elementwise = [&](int qt, const f32x4& S, const f32x4& dP, float (&pw)[4], float (&dsv)[4]) {
        const int q0 = 16 * qt + 4 * grp;
        const float4 l4 = *(const float4*)(&sLse2[q0]);
        const float4 w4 = *(const float4*)(&sW[q0]);
        const float4 c4 = *(const float4*)(&sWc[q0]);
        const int4 p4 = *(const int4*)(&sPos[ec][q0]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, wv[4] = {w4.x, w4.y, w4.z, w4.w};
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
        const int qp[4] = {p4.x, p4.y, p4.z, p4.w};
        if constexpr (!EXACT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool drop = CAUSAL ? (kpos >= qp[e]) : (kpos == qp[e]);
            const float p = drop ? 0.f : __builtin_amdgcn_exp2f(fmaf(S[e], ks2, -lv[e]));
            pw[e] = wv[e] * p;
            dsv[e] = p * fmaf(wv[e], dP[e], cv[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool self = kpos == qp[e];
            const bool drop = CAUSAL && kpos > qp[e];
            float p = __builtin_amdgcn_exp2f((self ? kSelf2 : S[e] * ks2) - lv[e]);
            if (lv[e] < kSelfOnly2) p = self ? (lv[e] > kSelfTwice2 ? 0.5f : 1.f) : 0.f;
            p = drop ? 0.f : p;
            pw[e] = wv[e] * p;
            const float dl = p * fmaf(wv[e], dP[e], cv[e]);
            dsv[e] = self ? 0.f : dl;
          }
        }
      };
      if constexpr (BF16) {
        const bf16x8 k0 = *(const bf16x8*)(&sX[sw][xoff(kr, grp)]);
        const bf16x8 k1 = *(const bf16x8*)(&sX[sw][xoff(kr, 4 + grp)]);
        const bf16x8 v0 = *(const bf16x8*)(&sV[sw][xoff(kr, grp)]);
        const bf16x8 v1 = *(const bf16x8*)(&sV[sw][xoff(kr, 4 + grp)]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x4 bp4[2], bs4[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int qt = 2 * ks + h;
            const int qr = 16 * qt + col;
            const bf16x8 q0 = *(const bf16x8*)(&sX[cur][xoff(qr, grp)]);
            const bf16x8 q1 = *(const bf16x8*)(&sX[cur][xoff(qr, 4 + grp)]);
            const bf16x8 d0 = *(const bf16x8*)(&sDO[xoff(qr, grp)]);
            const bf16x8 d1 = *(const bf16x8*)(&sDO[xoff(qr, 4 + grp)]);
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q0, k0, z, 0, 0, 0);
            const f32x4 S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1, k1, z, 0, 0, 0);
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = __builtin_amdgcn_mfma_f32_16x16x32_bf16(d0, v0, y, 0, 0, 0);
            const f32x4 dP = __builtin_amdgcn_mfma_f32_16x16x32_bf16(d1, v1, y, 0, 0, 0);
            float pw[4], dsv[4];
            elementwise(qt, S, dP, pw, dsv);
            bp4[h] = __builtin_convertvector((f32x4{pw[0], pw[1], pw[2], pw[3]}), bf16x4);
            bs4[h] = __builtin_convertvector((f32x4{dsv[0], dsv[1], dsv[2], dsv[3]}), bf16x4);
            const uint2 u = __builtin_bit_cast(
                uint2, __builtin_convertvector((f32x4{dsv[0] * kn, dsv[1] * kn, dsv[2] * kn, dsv[3] * kn}), bf16x4));
            dsk16[2 * qt] = u.x;
            dsk16[2 * qt + 1] = u.y;
          }
          // ---- dV^T += dO^T Pw, A^T += Xq^T dS (K = queries 32 ks .. 32 ks + 31, permuted;
          // rows = dims in tr_operand's order) ----
          const bf16x8 bp = __builtin_shufflevector(bp4[0], bp4[1], 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 bs = __builtin_shufflevector(bs4[0], bs4[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const bf16x8 ad = tr_operand(sDO, 32 * ks, dt, lane_v);
            const bf16x8 ax = tr_operand(sX[cur], 32 * ks, dt, lane_v);
            acc_v[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad, bp, acc_v[dt], 0, 0, 0);
            acc_a[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bs, acc_a[dt], 0, 0, 0);
          }
        }
      } else {
        // k-step s: lane group g feeds dim 16 g + s
        float kk[16], vv[16];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const float4 a = *(const float4*)(&sX[sw][kr * kXRow + 16 * grp + 4 * s4]);
          const float4 b = *(const float4*)(&sV[sw][kr * kXRow + 16 * grp + 4 * s4]);
          kk[4 * s4] = a.x; kk[4 * s4 + 1] = a.y; kk[4 * s4 + 2] = a.z; kk[4 * s4 + 3] = a.w;
          vv[4 * s4] = b.x; vv[4 * s4 + 1] = b.y; vv[4 * s4 + 2] = b.z; vv[4 * s4 + 3] = b.w;
        }
        float pw[4][4], dsv[4][4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const int qr = 16 * qt + col;
          f32x4 z = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const float4 a = *(const float4*)(&sX[cur][qr * kXRow + 16 * grp + 4 * s4]);
            const float4 b = *(const float4*)(&sDO[qr * kXRow + 16 * grp + 4 * s4]);
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              z = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], kk[4 * s4 + u], z, 0, 0, 0);
              y = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[u], vv[4 * s4 + u], y, 0, 0, 0);
            }
          }
          elementwise(qt, z, y, pw[qt], dsv[qt]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dskf[4 * qt + e] = dsv[qt][e] * kn;
        }
        // K index grp <-> query 16 qt + 4 grp + e, one MFMA per (qt, e)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qr = 16 * qt + 4 * grp + e;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const float ad = sDO[qr * kXRow + 16 * dt + col];
              const float ax = sX[cur][qr * kXRow + 16 * dt + col];
              acc_v[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, pw[qt][e], acc_v[dt], 0, 0, 0);
              acc_a[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ax, dsv[qt][e], acc_a[dt], 0, 0, 0);
            }
          }
      }
    };
    if (active) {
      if (sSelfOnly != 0) compute(std::true_type{});
      else compute(std::false_type{});
      if (!do_kv) zero_acc();  // look-back keys of the first step: not this run's
    }

    // ---- dQ^T = Xk^T (dS kn)^T for the current chunk's queries ----
    if (do_ds) {
      __syncthreads();  // every wave is done reading dO (the bf16 dS tile reuses its space)
      if (active) {
        if constexpr (BF16) {
          // The four lanes of a quad hold keys 4i .. 4i + 3, whose tile columns are
          // consecutive (permcol keeps a key's low two bits), for the same four
          // queries of each query tile.  A 4 x 4 transpose of their 16-bit values
          // inside the quad gives lane j the four keys of query j, written as one
          // 8-byte piece instead of four 2-byte stores to one word.
          const int j = lane_v & 3;
          const int kc0 = 64 * sw + (permcol(kr) & ~3);
          const uint32_t sel = (j & 1) ? 0x03020706u : 0x05040100u;
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
            const uint32_t d0 = dsk16[2 * qt], d1 = dsk16[2 * qt + 1];  // queries (0, 1), (2, 3) of key j
            // with lane j ^ 2: lanes 0, 1 keep queries 0-1 of keys j, j + 2; lanes 2, 3 queries 2-3
            const uint32_t got = quad_xor2((j & 2) ? d0 : d1);
            const uint32_t a = (j & 2) ? got : d0;  // key j & 1
            const uint32_t b = (j & 2) ? d1 : got;  // key (j & 1) + 2
            // with lane j ^ 1: the halves of query j of keys 0, 1 and of keys 2, 3
            const uint32_t a1 = quad_xor1(a), b1 = quad_xor1(b);
            uint2 w;
            w.x = __builtin_amdgcn_perm(a1, a, sel);
            w.y = __builtin_amdgcn_perm(b1, b, sel);
            *(uint2*)(&sDS16[voff(16 * qt + 4 * grp + j, kc0 >> 3) + (kc0 & 7)]) = w;
          }
        } else {
#pragma unroll
          for (int qt = 0; qt < 4; ++qt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sDsF[(16 * qt + 4 * grp + e) * kSRow + 64 * sw + kr] = dskf[4 * qt + e];
        }
      }
      __syncthreads();
      if (mine_cur) {
        // this wave's queries are its own key rows 16 kt + col of the current chunk
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int kp = 8 * (ks < 2 ? prv : cur) + 4 * (ks & 1) + grp;  // piece: columns 8 kp .. 8 kp + 7
            const bf16x8 bq = *(const bf16x8*)(&sDS16[voff(kr, kp)]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const bf16x8 a = tr_operand(sX[ks < 2 ? prv : cur], 32 * (ks & 1), dt, lane_v);
              acc_q[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq, acc_q[dt], 0, 0, 0);
            }
          }
        } else {
          // K index grp <-> key 4 (s & 15) + grp of slot (s < 16 ? prv : cur)
#pragma unroll 4
          for (int s = 0; s < 32; ++s) {
            const int sl = s < 16 ? prv : cur;
            const int kk = 4 * (s & 15) + grp;
            const float bq = sDsF[kr * kSRow + 64 * sl + kk];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const float a = sX[sl][kk * kXRow + 16 * dt + col];
              acc_q[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bq, acc_q[dt], 0, 0, 0);
            }
          }
        }
      }
    }

    // ---- the previous chunk's keys are complete: dx = dq + kn (a - khat (khat . a)), dv ----
    if (!mine_cur && c > c0) {
      const int chunk = (c - 1 + n_chunks) % n_chunks;
      const float kn = sKn[sw][kr];
      const bool tiny = kn > 0.12e12f;  // |x| at the 1e-12 floor: khat = x / 1e-12, no projection
      // bf16: accumulator row 4 grp + e of tile dt is dim 32 (dt >> 1) + 8 grp + 4 (dt & 1) + e
      // (tr_operand), so tiles 2h and 2h + 1 hold piece 4h + grp of the key's row: its dim
      // 32 h + 8 grp + u is element u & 3 of tile 2h + (u >> 2).  fp32: tile dt holds dims
      // 16 dt + 4 grp + e.
      float xv[4][4];
      if constexpr (BF16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint4 r = *(const uint4*)(&sX[sw][xoff(kr, 4 * h + grp)]);
          const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[2 * h + (e >> 1)][2 * (e & 1)] = bf_lo(rw[e]);
            xv[2 * h + (e >> 1)][2 * (e & 1) + 1] = bf_hi(rw[e]);
          }
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const float4 r = *(const float4*)(&sX[sw][kr * kXRow + 16 * dt + 4 * grp]);
          xv[dt][0] = r.x; xv[dt][1] = r.y; xv[dt][2] = r.z; xv[dt][3] = r.w;
        }
      }
      // x . a over the lane's 16 dims; bf16 in the order 8 grp + 2e, 32 + 8 grp + 2e,
      // 8 grp + 2e + 1, 32 + 8 grp + 2e + 1 (e = 0..3), fp32 tile by tile
      float dot = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = BF16 ? 2 * (s2 & 1) + (e >> 1) : s2;
          const int u = BF16 ? 2 * (e & 1) + (s2 >> 1) : e;
          dot = fmaf(xv[t][u], acc_a[t][u], dot);
        }
      // sum over the 4 lanes holding this key (lanes l, l^16, l^32, l^48)
      {
        auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
        dot = __uint_as_float(h[0]) + __uint_as_float(h[1]);
        auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(dot), __float_as_uint(dot), false, false);
        dot = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      }
      // khat = 8 kn x, so khat (khat . a) = 64 kn^2 x (x . a)
      const float proj = tiny ? 0.f : 64.f * kn * kn * dot;
      const size_t row = (size_t)chunk * kChunk + kr;
      if constexpr (BF16) {
        // word e of piece h: dims 32 h + 8 grp + 2e, + 1: elements 2 (e & 1), + 1 of tile 2h + (e >> 1)
        uint32_t rx[2][4], rv[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 2 * h + (e >> 1), u = 2 * (e & 1);
            const float x0 = acc_q[t][u] + kn * (acc_a[t][u] - proj * xv[t][u]);
            const float x1 = acc_q[t][u + 1] + kn * (acc_a[t][u + 1] - proj * xv[t][u + 1]);
            rx[h][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
            rv[h][e] = __builtin_bit_cast(uint32_t,
                                          __builtin_convertvector(f32x2{acc_v[t][u], acc_v[t][u + 1]}, bf16x2));
          }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 px = {rx[h][0], rx[h][1], rx[h][2], rx[h][3]}, pv = {rv[h][0], rv[h][1], rv[h][2], rv[h][3]};
          u32x4* const qx = (u32x4*)(dxb + row * kD + 32 * h + 8 * grp);
          u32x4* const qv = (u32x4*)(dvb + row * kD + 32 * h + 8 * grp);
          if constexpr (NT) {
            __builtin_nontemporal_store(px, qx);
            __builtin_nontemporal_store(pv, qv);
          } else {
            *qx = px;
            *qv = pv;
          }
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          float ox[4], ov[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ox[e] = acc_q[dt][e] + kn * (acc_a[dt][e] - proj * xv[dt][e]);
            ov[e] = acc_v[dt][e];
          }
          const f32x4 px = {ox[0], ox[1], ox[2], ox[3]}, pv = {ov[0], ov[1], ov[2], ov[3]};
          f32x4* const qx = (f32x4*)(dxb + row * kD + 16 * dt + 4 * grp);
          f32x4* const qv = (f32x4*)(dvb + row * kD + 16 * dt + 4 * grp);
          if constexpr (NT) {
            __builtin_nontemporal_store(px, qx);
            __builtin_nontemporal_store(pv, qv);
          } else {
            *qx = px;
            *qv = pv;
          }
        }
      }
      zero_acc();
    }

    __syncthreads();  // every wave is done with slot prv, dO and the dS tile
    if (c < c1) {
      commit(prv, true);  // step c+1: its keys in slot (c+1) & 1 = prv, its queries
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// bwd_reduce: dx_i = sum_r dx_slot[undo_r(i)], dv_i likewise; 8 lanes (bf16) or
// 16 lanes (fp32) per token, 16 bytes each.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const void* __restrict__ dx_slot,
                                                         const void* __restrict__ dv_slot,
                                                         const int32_t* __restrict__ undo_idx, void* __restrict__ dx,
                                                         void* __restrict__ dv, int L, int n_h, size_t n_tokens,
                                                         bool nt_in) {
  constexpr int kLanesPerTok = BF16 ? 8 : 16;
  constexpr int kE = BF16 ? 8 : 4;
  constexpr size_t kEs = BF16 ? 2 : 4;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t tok = gid / kLanesPerTok;
  const int sub = (int)(gid % kLanesPerTok);
  if (tok >= n_tokens) return;
  const size_t bh = tok / L;
  const int i = (int)(tok % L);
  const size_t n_slots = (size_t)n_h * L;
  const int32_t* u = undo_idx + bh * n_slots + i;
  int g[kMaxHashes];
#pragma unroll
  for (int r = 0; r < kMaxHashes; ++r)
    if (r < n_h) g[r] = (int)min((uint32_t)u[(size_t)r * L], (uint32_t)(n_slots - 1));
  uint4 rx[kMaxHashes], rv[kMaxHashes];
#pragma unroll
  for (int r = 0; r < kMaxHashes; ++r)
    if (r < n_h) {
      const size_t off = ((bh * n_slots + g[r]) * kD) * kEs + 16 * sub;
      if (nt_in) {  // rows the attention backward streamed past the last-level cache
        const u32x4 tx = __builtin_nontemporal_load((const u32x4*)((const char*)dx_slot + off));
        const u32x4 tv = __builtin_nontemporal_load((const u32x4*)((const char*)dv_slot + off));
        rx[r] = make_uint4(tx[0], tx[1], tx[2], tx[3]);
        rv[r] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
      } else {
        rx[r] = *(const uint4*)((const char*)dx_slot + off);
        rv[r] = *(const uint4*)((const char*)dv_slot + off);
      }
    }
  float ax[kE], av[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) ax[e] = av[e] = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxHashes; ++r)
    if (r < n_h) {
      const uint32_t wx[4] = {rx[r].x, rx[r].y, rx[r].z, rx[r].w};
      const uint32_t wv[4] = {rv[r].x, rv[r].y, rv[r].z, rv[r].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (BF16) {
          ax[2 * k] += bf_lo(wx[k]);
          ax[2 * k + 1] += bf_hi(wx[k]);
          av[2 * k] += bf_lo(wv[k]);
          av[2 * k + 1] += bf_hi(wv[k]);
        } else {
          ax[k] += __uint_as_float(wx[k]);
          av[k] += __uint_as_float(wv[k]);
        }
      }
    }
  const size_t off = (tok * kD) * kEs + 16 * sub;
  if constexpr (BF16) {
    uint4 ox, ov;
    uint32_t px[4], pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      px[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{ax[2 * k], ax[2 * k + 1]}, bf16x2));
      pv[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{av[2 * k], av[2 * k + 1]}, bf16x2));
    }
    ox = make_uint4(px[0], px[1], px[2], px[3]);
    ov = make_uint4(pv[0], pv[1], pv[2], pv[3]);
    *(uint4*)((char*)dx + off) = ox;
    *(uint4*)((char*)dv + off) = ov;
  } else {
    *(float4*)((char*)dx + off) = make_float4(ax[0], ax[1], ax[2], ax[3]);
    *(float4*)((char*)dv + off) = make_float4(av[0], av[1], av[2], av[3]);
  }
}

}  // namespace

hipError_t launch_bwd_prep(const void* qk, const void* out, const void* dout, const float* dlse,
                           const float* lse_sorted, const int32_t* undo_idx, float2* tok_w, float2* tok_scale,
                           int BH, int L, int n_h, lsh_dtype dt, hipStream_t s) {
  const size_t n_tok = (size_t)BH * L;
  const unsigned grid = (unsigned)((n_tok + 15) / 16);
  if (dt == LSH_BF16)
    bwd_prep_kernel<true><<<grid, 256, 0, s>>>(qk, out, dout, dlse, lse_sorted, undo_idx, tok_w, tok_scale, L, n_h,
                                               n_tok);
  else
    bwd_prep_kernel<false><<<grid, 256, 0, s>>>(qk, out, dout, dlse, lse_sorted, undo_idx, tok_w, tok_scale, L,
                                                n_h, n_tok);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* qk, const void* v, const void* dout, const int32_t* sorted_idx,
                           const float* lse_sorted, const float2* tok_w, const float2* tok_scale, void* dx_slot,
                           void* dv_slot, int BH, int L, int n_h, int causal, lsh_dtype dt, hipStream_t s) {
  const int n_slots = n_h * L;
  const int n_chunks = n_slots / kChunk;
  const int blocks_per_bh = (n_chunks + kBwdChunksPerBlock - 1) / kBwdChunksPerBlock;
  const unsigned grid = (unsigned)blocks_per_bh * (unsigned)BH;
  const bool nt = stream_slot_rows(BH, L, n_h, dt);
#define LSH_BWD_LAUNCH(B16, CA)                                                                               \
  (nt ? attn_bwd_kernel<B16, CA, true> : attn_bwd_kernel<B16, CA, false>)<<<grid, 512, 0, s>>>(              \
      (const typename BwdTraits<B16>::T*)qk, (const typename BwdTraits<B16>::T*)v,                           \
      (const typename BwdTraits<B16>::T*)dout, sorted_idx, lse_sorted, tok_w, tok_scale,                     \
      (typename BwdTraits<B16>::T*)dx_slot, (typename BwdTraits<B16>::T*)dv_slot, L, n_h, n_slots, n_chunks, \
      blocks_per_bh)
  if (dt == LSH_BF16) {
    if (causal) LSH_BWD_LAUNCH(true, true);
    else LSH_BWD_LAUNCH(true, false);
  } else {
    if (causal) LSH_BWD_LAUNCH(false, true);
    else LSH_BWD_LAUNCH(false, false);
  }
#undef LSH_BWD_LAUNCH
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const void* dx_slot, const void* dv_slot, const int32_t* undo_idx, void* dx, void* dv,
                             int BH, int L, int n_h, lsh_dtype dt, hipStream_t s) {
  const size_t n_tok = (size_t)BH * L;
  const int lanes = dt == LSH_BF16 ? 8 : 16;
  const unsigned grid = (unsigned)((n_tok * lanes + 255) / 256);
  const bool nt = stream_slot_rows(BH, L, n_h, dt);  // as attn_bwd wrote them
  if (dt == LSH_BF16)
    bwd_reduce_kernel<true><<<grid, 256, 0, s>>>(dx_slot, dv_slot, undo_idx, dx, dv, L, n_h, n_tok, nt);
  else
    bwd_reduce_kernel<false><<<grid, 256, 0, s>>>(dx_slot, dv_slot, undo_idx, dx, dv, L, n_h, n_tok, nt);
  return hipGetLastError();
}

}  // namespace lsh
