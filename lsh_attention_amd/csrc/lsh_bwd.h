// Internal declarations of the backward kernels (attn_bwd.hip).
#pragma once

#include "lsh_internal.h"

namespace lsh {

// Per token: combine weights w of its n_h rounds and w (dLSE_i - dout_i . out_i)
// (tok_w, [BH][L][n_h]); key scales (log2(e) kn, kn) per token (tok_scale,
// [BH][L]), kn = 1 / (8 max(|x|, 1e-12)).  dlse may be null.
hipError_t launch_bwd_prep(const void* qk, const void* out, const void* dout, const float* dlse,
                           const float* lse_sorted, const int32_t* undo_idx, float2* tok_w,
                           float2* tok_scale, int BH, int L, int n_h, lsh_dtype dt, hipStream_t s);
// Per slot: the finished query + key role gradient of x and the value gradient
// ([BH][n_h*L][64] each, element type dt).
hipError_t launch_attn_bwd(const void* qk, const void* v, const void* dout, const int32_t* sorted_idx,
                           const float* lse_sorted, const float2* tok_w, const float2* tok_scale,
                           void* dx_slot, void* dv_slot, int BH, int L, int n_h, int causal, lsh_dtype dt,
                           hipStream_t s);
// Per token: the sums of its n_h slots' rows.
hipError_t launch_bwd_reduce(const void* dx_slot, const void* dv_slot, const int32_t* undo_idx, void* dx,
                             void* dv, int BH, int L, int n_h, lsh_dtype dt, hipStream_t s);

}  // namespace lsh
