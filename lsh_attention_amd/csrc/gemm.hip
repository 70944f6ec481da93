// Dense parts of one reversible Reformer block around the LSH attention: the
// projections and the feed-forward are GEMMs with fused epilogues, plus a row
// LayerNorm.
//
// Reformer explainer (akshathtiwari.co.in/blog/reformer) and Reformer
// abstract: reversible residual layers and a chunked feed-forward are the
// memory savings that, with LSH attention, fit about 64K tokens on one
// accelerator.  The block is y1 = x1 + F(x2), y2 = x2 + G(y1) with F the
// attention sublayer (LayerNorm, shared-QK and V projections, LSH attention
// per head, output projection) and G the feed-forward sublayer (LayerNorm,
// Linear(dim, 4 dim) + bias, GELU, Linear(4 dim, dim) + bias), G taken over
// chunks of rows.
//
// gfx950 GEMM: C[M x N] = A[M x K] . W^T with W stored [N x K] (a Linear
// layer's layout, both operands contiguous in K), bf16 in, fp32 accumulate,
// bf16 out.  128 x 128 tiles, 4 waves of 64 x 64 on v_mfma_f32_16x16x32_bf16,
// K staged 64 at a time through double-buffered LDS (unpadded 128-byte rows
// whose 16-byte pieces are XOR-swizzled by the row, so the operand reads and
// the staging writes run at the full LDS rate), one barrier per stage; two
// register sets keep the global loads two stages ahead of the MFMAs.  The
// epilogue stages the fp32 tile in LDS and writes 16-byte row pieces.
// Tiles are ordered so that all column tiles of a row tile run on one XCD (its
// A rows are fetched into one L2).  Epilogue: + bias, GELU, + residual, and the
// attention's head-major layout [B][H][L][64] on input (A) or output (C).
#include <type_traits>

#include "lsh_block.h"

namespace lsh {

namespace {

constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kRow = 64;        // LDS operand row: 64 bf16
constexpr int kCRow = kTN + 4;  // epilogue fp32 row
constexpr int kOpBytes = 2 * (kTM + kTN) * kRow * 2;  // both operands, double-buffered
constexpr int kSmemBytes = kOpBytes > kTM * kCRow * 4 ? kOpBytes : kTM * kCRow * 4;

// Operand LDS element offset of (row, 16-byte piece): piece p of row r sits at
// p ^ (r mod 8).  16 lanes reading 16 rows with the 4 lane groups on 4 pieces
// (the MFMA operand pattern) run at full rate in this layout; rows padded to
// 144 bytes measured 1.6x slower for them on gfx950.
__device__ inline int soff(int row, int piece) { return row * kRow + 8 * (piece ^ (row & 7)); }

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ inline float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, with erf from Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26: for z >= 0,
// erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2), t = 1 / (1 + p z),
// absolute error at most 1.5e-7 (far below bf16 rounding); erf is odd.
__device__ inline float gelu_as(float x) {
  constexpr float p = 0.3275911f, a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f,
                  a4 = -1.453152027f, a5 = 1.061405429f;
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(p, z, 1.f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
  const float e = __builtin_amdgcn_exp2f(-z * z * 1.4426950408889634f);
  const float erf_abs = fmaf(-poly, e, 1.f);
  return 0.5f * x * (1.f + copysignf(erf_abs, x));
}

// element offset of (row m, column k) of a [M x K] operand in the given layout
template <int MODE>
__device__ inline size_t ofs(int m, int k, int K, int L, int H) {
  if constexpr (MODE == kLayoutRows) {
    return (size_t)m * K + k;
  } else {  // head-major [B][H][L][64], m = b L + l, k = 64 h + d
    const int b = m / L, l = m - b * L;
    return (((size_t)b * H + (k >> 6)) * L + l) * 64 + (k & 63);
  }
}

template <int AMODE, int CMODE, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ bias,
                                                      const uint16_t* __restrict__ resid, uint16_t* __restrict__ C,
                                                      int M, int N, int K, int L, int H, int n_items) {
  // [A buf 0][A buf 1][W buf 0][W buf 1]; the epilogue reuses it as one fp32 tile
  __shared__ __attribute__((aligned(16))) uint16_t sBuf[kSmemBytes / 2];
  uint16_t* const sA0 = sBuf;
  uint16_t* const sW0 = sBuf + 2 * kTM * kRow;
  const unsigned item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= (unsigned)n_items) return;
  const int n_tiles = N / kTN;
  const int m0 = (int)(item / n_tiles) * kTM, n0 = (int)(item % n_tiles) * kTN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> LDS: 128 rows x 8 pieces of 16 bytes per operand; thread t moves
  // pieces t + 256 i (row p >> 3, piece p & 7).  Two register sets: stage k+2 is
  // loaded while stage k is computed and stage k+1 waits in the other set, so a
  // load has two stages of MFMA work to arrive.
  uint4 ra0[4], rw0[4], ra1[4], rw1[4];  // the two register sets (compile-time selected)
  // A element offsets of this thread's 4 rows at k = 8 (p & 7); per stage only
  // k0 (a multiple of 64) is added: + k0 in the rows layout, + (k0 / 64) L 64 in
  // the head-major one.  Rows past M (a partial last row tile) read row M - 1:
  // they only feed output rows that are never stored, and the loads stay
  // unconditional.
  size_t abase[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = tid + 256 * i;
    abase[i] = ofs<AMODE>(min(m0 + (p >> 3), M - 1), 8 * (p & 7), K, L, H);
  }
  const size_t astep = AMODE == kLayoutRows ? (size_t)kTK : (size_t)L * 64;  // per stage of 64 columns
  auto load = [&](auto set, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, r = p >> 3, pc = p & 7;
      const uint4 va = *(const uint4*)(A + abase[i] + (size_t)(k0 / kTK) * astep);
      const uint4 vw = *(const uint4*)(W + (size_t)(n0 + r) * K + k0 + 8 * pc);
      if constexpr (decltype(set)::value == 0) {
        ra0[i] = va;
        rw0[i] = vw;
      } else {
        ra1[i] = va;
        rw1[i] = vw;
      }
    }
  };
  auto store = [&](auto set, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + 256 * i, r = p >> 3, pc = p & 7;
      const uint4 va = decltype(set)::value == 0 ? ra0[i] : ra1[i];
      const uint4 vw = decltype(set)::value == 0 ? rw0[i] : rw1[i];
      *(uint4*)(&sA0[buf * kTM * kRow + soff(r, pc)]) = va;
      *(uint4*)(&sW0[buf * kTN * kRow + soff(r, pc)]) = vw;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *(const bf16x8*)(&sA0[buf * kTM * kRow + soff(64 * wm + 16 * i + col, 4 * s + grp)]);
        b[i] = *(const bf16x8*)(&sW0[buf * kTN * kRow + soff(64 * wn + 16 * i + col, 4 * s + grp)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int nk = K / kTK;
  load(S0{}, 0);
  if (nk > 1) load(S1{}, kTK);
  store(S0{}, 0);
  __syncthreads();
  // stage k: compute buffer k & 1; set k & 1 is free once stage k is in LDS
  auto step = [&](int kb, auto set, auto other) {
    constexpr int sv = decltype(set)::value;
    if (kb + 2 < nk) load(set, (kb + 2) * kTK);
    compute(sv);
    if (kb + 1 < nk) store(other, sv ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  };
  for (int kb = 0; kb < nk; kb += 2) {
    step(kb, S0{}, S1{});
    if (kb + 1 < nk) step(kb + 1, S1{}, S0{});
  }

  // ---- epilogue through LDS: lane holds C[64 wm + 16 i + 4 grp + e][64 wn + 16 j + col].
  // The fp32 tile (+ bias, GELU) is staged in LDS and written as 16-byte row
  // pieces, the residual added before the one rounding to bf16.
  float* const sC = (float*)sBuf;  // [128][kCRow] fp32, over the operand buffers
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nl = 64 * wn + 16 * j + col;
    const float bv = (EPI & kEpiBias) ? from_bf16(bias[n0 + nl]) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = acc[i][j][e] + bv;
        if constexpr ((EPI & kEpiGelu) != 0) x = gelu_as(x);
        sC[(64 * wm + 16 * i + 4 * grp + e) * kCRow + nl] = x;
      }
  }
  __syncthreads();
  // 128 rows x 16 pieces of 8 columns: thread t writes pieces t + 256 i
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = tid + 256 * i, ml = p >> 4, pc = p & 15;
    const int m = m0 + ml, n = n0 + 8 * pc;
    if (m >= M) continue;
    const float4 lo = *(const float4*)(&sC[ml * kCRow + 8 * pc]);
    const float4 hi = *(const float4*)(&sC[ml * kCRow + 8 * pc + 4]);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    if constexpr ((EPI & kEpiResid) != 0) {
      const uint4 r = *(const uint4*)(resid + (size_t)m * N + n);
      const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] += bf_lo(rr[k]);
        v[2 * k + 1] += bf_hi(rr[k]);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (uint32_t)to_bf16(v[2 * k]) | ((uint32_t)to_bf16(v[2 * k + 1]) << 16);
    *(uint4*)(C + ofs<CMODE>(m, n, N, L, H)) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// LayerNorm over rows of `dim` (a multiple of 8, at most 1024): one wave per
// row, each lane 16-byte pieces lane, lane + 64; two-pass mean / variance in fp32.
__global__ __launch_bounds__(256) void layer_norm_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ g,
                                                         const uint16_t* __restrict__ b, uint16_t* __restrict__ y,
                                                         int rows, int dim) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves leave together
  const int pieces = dim >> 3;
  const uint16_t* xr = x + (size_t)row * dim;
  float v[2][8];
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = lane + 64 * u;
    if (p < pieces) {
      const uint4 w = *(const uint4*)(xr + 8 * p);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[u][2 * k] = bf_lo(ww[k]);
        v[u][2 * k + 1] = bf_hi(ww[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[u][k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[u][k];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
  const float mean = s / (float)dim;
  float q = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (lane + 64 * u < pieces)
#pragma unroll
      for (int k = 0; k < 8; ++k) q = fmaf(v[u][k] - mean, v[u][k] - mean, q);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) q += __shfl_xor(q, o);
  const float rstd = 1.0f / __builtin_sqrtf(q / (float)dim + 1e-5f);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int p = lane + 64 * u;
    if (p >= pieces) continue;
    const uint4 gw = *(const uint4*)(g + 8 * p), bw = *(const uint4*)(b + 8 * p);
    const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w}, bb[4] = {bw.x, bw.y, bw.z, bw.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float y0 = (v[u][2 * k] - mean) * rstd * bf_lo(gg[k]) + bf_lo(bb[k]);
      const float y1 = (v[u][2 * k + 1] - mean) * rstd * bf_hi(gg[k]) + bf_hi(bb[k]);
      o[k] = (uint32_t)to_bf16(y0) | ((uint32_t)to_bf16(y1) << 16);
    }
    *(uint4*)(y + (size_t)row * dim + 8 * p) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <int AMODE, int CMODE>
hipError_t launch_gemm_t(const void* A, const void* W, const void* bias, const void* resid, void* C, int M, int N,
                         int K, int L, int H, int epi, hipStream_t s) {
  const int items = ((M + kTM - 1) / kTM) * (N / kTN);
  const unsigned grid = xcd_grid((unsigned)items);
  const auto* a = (const uint16_t*)A;
  const auto* w = (const uint16_t*)W;
  const auto* bi = (const uint16_t*)bias;
  const auto* re = (const uint16_t*)resid;
  auto* c = (uint16_t*)C;
  switch (epi) {
    case 0: gemm_kernel<AMODE, CMODE, 0><<<grid, 256, 0, s>>>(a, w, bi, re, c, M, N, K, L, H, items); break;
    case kEpiBias | kEpiGelu:
      gemm_kernel<AMODE, CMODE, kEpiBias | kEpiGelu><<<grid, 256, 0, s>>>(a, w, bi, re, c, M, N, K, L, H, items);
      break;
    case kEpiResid:
      gemm_kernel<AMODE, CMODE, kEpiResid><<<grid, 256, 0, s>>>(a, w, bi, re, c, M, N, K, L, H, items);
      break;
    case kEpiBias | kEpiResid:
      gemm_kernel<AMODE, CMODE, kEpiBias | kEpiResid><<<grid, 256, 0, s>>>(a, w, bi, re, c, M, N, K, L, H, items);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const void* A, int a_layout, const void* W, const void* bias, const void* resid, void* C,
                       int c_layout, int M, int N, int K, int L, int H, int epi, hipStream_t s) {
  if (N % kTN != 0 || K % kTK != 0) return hipErrorInvalidValue;
  if (a_layout == kLayoutRows && c_layout == kLayoutRows)
    return launch_gemm_t<kLayoutRows, kLayoutRows>(A, W, bias, resid, C, M, N, K, L, H, epi, s);
  if (a_layout == kLayoutRows && c_layout == kLayoutHeads)
    return launch_gemm_t<kLayoutRows, kLayoutHeads>(A, W, bias, resid, C, M, N, K, L, H, epi, s);
  if (a_layout == kLayoutHeads && c_layout == kLayoutRows)
    return launch_gemm_t<kLayoutHeads, kLayoutRows>(A, W, bias, resid, C, M, N, K, L, H, epi, s);
  return hipErrorInvalidValue;
}

hipError_t launch_layer_norm(const void* x, const void* g, const void* b, void* y, int rows, int dim, hipStream_t s) {
  if (dim % 8 != 0 || dim > 1024) return hipErrorInvalidValue;
  layer_norm_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)g,
                                                                 (const uint16_t*)b, (uint16_t*)y, rows, dim);
  return hipGetLastError();
}

}  // namespace lsh
