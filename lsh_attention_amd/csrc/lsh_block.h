// Internal declarations of the dense kernels of the reversible block (gemm.hip).
#pragma once

#include "lsh_internal.h"

namespace lsh {

// Operand layouts: [M x K] rows, or the attention's head-major [B][H][L][64]
// with m = b L + l and k = 64 h + d (K = 64 H).
constexpr int kLayoutRows = 0;
constexpr int kLayoutHeads = 1;
// Epilogue bits: + bias[n], then GELU, then + resid[m][n] (rows layout).
constexpr int kEpiBias = 1;
constexpr int kEpiGelu = 2;
constexpr int kEpiResid = 4;

// C = epilogue(A . W^T), W [N x K] (a Linear layer's [out x in]); bf16 in and out,
// fp32 accumulation.  N % 128 == 0, K % 64 == 0; any M.  Supported layout pairs:
// rows -> rows, rows -> heads, heads -> rows; epilogues 0, bias|gelu, resid,
// bias|resid.
hipError_t launch_gemm(const void* A, int a_layout, const void* W, const void* bias, const void* resid, void* C,
                       int c_layout, int M, int N, int K, int L, int H, int epi, hipStream_t s);
// y = (x - mean) / sqrt(var + 1e-5) * g + b over rows of dim (dim % 8 == 0, <= 1024), bf16.
hipError_t launch_layer_norm(const void* x, const void* g, const void* b, void* y, int rows, int dim, hipStream_t s);

}  // namespace lsh
