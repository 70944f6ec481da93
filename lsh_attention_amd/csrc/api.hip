// C ABI of the shared-QK LSH attention forward pass: argument validation,
// workspace carving and the stream-ordered launch sequence.  Validation runs
// entirely on the host and returns before anything is enqueued.
#include <string.h>

#include <mutex>
#include <vector>

#include "lsh_block.h"
#include "lsh_bwd.h"

using namespace lsh;

namespace {

constexpr size_t kAlign = 256;

size_t elem_size(lsh_dtype dt) { return dt == LSH_BF16 ? 2 : 4; }

bool dtype_ok(lsh_dtype dt) { return dt == LSH_F32 || dt == LSH_BF16; }

bool attend_ok(int attend) { return (attend & ~(LSH_ATTEND_SAME_BUCKET | LSH_ATTEND_DEDUP)) == 0; }

// B, H or L == 0 is a valid, empty problem: the entry points return LSH_OK at
// once, with no pointer checked and nothing enqueued (workspace size 0).
bool is_empty(int B, int H, int L) { return B == 0 || H == 0 || L == 0; }

int check_problem(int B, int H, int L, int D, int n_h) {
  if (B < 0 || H < 0 || L < 0 || D <= 0 || n_h <= 0) return LSH_ERR_SHAPE;
  if (D != kD) return LSH_ERR_UNSUPPORTED;
  if (n_h > kMaxHashes) return LSH_ERR_UNSUPPORTED;
  if (L % kChunk != 0 || L > kMaxLen) return LSH_ERR_SHAPE;
  const uint64_t slots = (uint64_t)B * (uint64_t)H * (uint64_t)n_h * (uint64_t)L;
  if (slots > 0x7FFFFFFFull) return LSH_ERR_SHAPE;
  return LSH_OK;
}

int check_buckets(int n_b, int L) {
  if (n_b < 1 || n_b > kMaxBuckets) return LSH_ERR_BUCKETS;
  if (n_b > 1 && (n_b % 2) != 0) return LSH_ERR_BUCKETS;
  if ((uint64_t)n_b * (uint64_t)sort_tiles(L, n_b) > 0x7FFFFFFFull) return LSH_ERR_SHAPE;
  return LSH_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Sequential carving of a workspace into 256-byte aligned regions.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  }
};

struct HashWs {
  size_t rot_t, colmax, fix_count, fix_queue, total;
};
HashWs hash_ws(int BH, int L, int n_b, int n_h, lsh_dtype dt) {
  Carver c;
  HashWs w;
  w.rot_t = c.take((size_t)n_h * padded_half(n_b) * kD * elem_size(dt));
  w.colmax = c.take((size_t)n_h * colmax_blocks(n_b) * sizeof(float));
  w.fix_count = c.take(sizeof(int));
  w.fix_queue = c.take((size_t)BH * n_h * L * sizeof(int));
  w.total = c.off;
  return w;
}

size_t sort_ws_bytes(int BH, int L, int n_b, int n_h) {
  return align_up((size_t)BH * n_h * n_b * sort_tiles(L, n_b) * sizeof(int), kAlign);
}

struct FwdWs {
  HashWs hash;
  size_t hash_base, sort_base, buckets, sorted_idx, undo_idx, o_sorted, lse_sorted, token_scales, tok_rec, total;
};
FwdWs fwd_ws(int BH, int L, int n_b, int n_h, lsh_dtype dt) {
  Carver c;
  FwdWs w;
  const size_t slots = (size_t)BH * n_h * L;
  w.hash = hash_ws(BH, L, n_b, n_h, dt);
  w.hash_base = c.take(w.hash.total);  // first: lsh_hash_uncertified reads it at offset 0
  w.sort_base = c.take(sort_ws_bytes(BH, L, n_b, n_h));
  w.buckets = c.take(slots * sizeof(int32_t));
  w.sorted_idx = c.take(slots * sizeof(int32_t));
  w.undo_idx = c.take(slots * sizeof(int32_t));
  w.o_sorted = c.take(slots * kD * elem_size(dt));
  w.lse_sorted = c.take(slots * sizeof(float));
  w.token_scales = c.take((size_t)BH * L * sizeof(float2));
  w.tok_rec = c.take(slots * sizeof(int32_t));  // set-union variant only
  w.total = c.off;
  return w;
}

struct BwdWs {
  size_t tok_w, tok_scale, dx_slot, dv_slot, total;
};
BwdWs bwd_ws(int BH, int L, int n_h, lsh_dtype dt) {
  Carver c;
  BwdWs w;
  const size_t slots = (size_t)BH * n_h * L;
  w.tok_w = c.take(slots * sizeof(float2));
  w.tok_scale = c.take((size_t)BH * L * sizeof(float2));
  w.dx_slot = c.take(slots * kD * elem_size(dt));
  w.dv_slot = c.take(slots * kD * elem_size(dt));
  w.total = c.off;
  return w;
}

struct BlockWs {
  FwdWs attn;
  size_t h1, qk, v, att, attn_base, h2, hid, total;
};
BlockWs block_ws(int B, int L, int heads, int n_b, int n_h, int chunk_rows) {
  Carver c;
  BlockWs w;
  const size_t M = (size_t)B * L, dim = (size_t)heads * kD;
  const size_t rows = chunk_rows > 0 ? (size_t)chunk_rows : M;
  w.attn = fwd_ws(B * heads, L, n_b, n_h, LSH_BF16);
  w.h1 = c.take(M * dim * 2);
  w.qk = c.take(M * dim * 2);
  w.v = c.take(M * dim * 2);
  w.att = c.take(M * dim * 2);
  w.attn_base = c.take(w.attn.total);
  w.h2 = c.take(M * dim * 2);
  w.hid = c.take((rows < M ? rows : M) * 4 * dim * 2);
  w.total = c.off;
  return w;
}

int check_block(int B, int L, int heads, int n_b, int n_h, int chunk_len, int chunk_rows, lsh_dtype dt) {
  int st = check_problem(B, heads, L, kD, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st != LSH_OK) return st;
  if (chunk_len != kChunk) return chunk_len <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (chunk_rows < 0) return LSH_ERR_SHAPE;
  if (dt != LSH_BF16 || heads % 2 != 0 || heads > 16) return LSH_ERR_UNSUPPORTED;
  if ((uint64_t)B * L * heads * kD * 4 > 0x7FFFFFFFull) return LSH_ERR_SHAPE;
  return LSH_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LSH_OK : LSH_ERR_HIP; }

// Records stage event k of `ev` on s; a NULL array or a NULL entry records nothing.
hipError_t record_stage(void* const* ev, int k, hipStream_t s) {
  return ev == nullptr || ev[k] == nullptr ? hipSuccess : hipEventRecord((hipEvent_t)ev[k], s);
}

// Enqueue hashing (prep, MFMA hash, fixup) into the given scratch regions.
hipError_t enqueue_hash(const void* qk, const void* rot, int32_t* buckets, float2* token_scales, char* ws,
                        const HashWs& w, int BH, int L, int n_b, int n_h, lsh_dtype dt, hipStream_t s,
                        void* const* ev, int* k) {
  auto mark = [&](void) -> hipError_t {
    if (ev == nullptr) return hipSuccess;
    ++*k;
    return record_stage(ev, *k, s);
  };
  hipError_t e;
  if (n_b == 1) {
    if ((e = launch_fill_zero(buckets, (size_t)BH * n_h * L, s)) != hipSuccess) return e;
    if ((e = mark()) != hipSuccess) return e;
    if ((e = mark()) != hipSuccess) return e;
    return mark();
  }
  float* colmax = (float*)(ws + w.colmax);
  int* count = (int*)(ws + w.fix_count);
  int* queue = (int*)(ws + w.fix_queue);
  void* rot_t = ws + w.rot_t;
  if ((e = launch_prep(rot, rot_t, colmax, count, n_h, n_b, dt, s)) != hipSuccess) return e;
  if ((e = mark()) != hipSuccess) return e;
  if ((e = launch_hash(qk, rot_t, colmax, buckets, queue, count, token_scales, BH, L, n_b, n_h, dt, s)) !=
      hipSuccess)
    return e;
  if ((e = mark()) != hipSuccess) return e;
  if ((e = launch_fixup(qk, rot_t, colmax, buckets, queue, count, L, n_b, n_h, dt, s)) != hipSuccess) return e;
  return mark();
}

hipError_t enqueue_sort(const int32_t* buckets, int32_t* sorted_idx, int32_t* undo_idx, int* hist, int BH, int L,
                        int n_b, int n_h, hipStream_t s, void* const* ev, int* k) {
  auto mark = [&](void) -> hipError_t {
    if (ev == nullptr) return hipSuccess;
    ++*k;
    return record_stage(ev, *k, s);
  };
  const int BHR = BH * n_h;
  hipError_t e;
  if ((e = launch_sort_hist(buckets, hist, BHR, L, n_b, s)) != hipSuccess) return e;
  if ((e = mark()) != hipSuccess) return e;
  if ((e = launch_sort_scatter(buckets, hist, sorted_idx, undo_idx, BHR, L, n_b, n_h, s)) != hipSuccess) return e;
  return mark();
}

}  // namespace

namespace lsh {
namespace {
// Dependent FMAs between two reads of the shader-cycle and real-time counters.
__global__ __launch_bounds__(256) void clock_spin_kernel(unsigned long long* __restrict__ ticks, int iters) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  float a = (float)threadIdx.x * 1e-3f, b = 1.0001f;
  for (int i = 0; i < iters; ++i) {
    a = fmaf(a, b, 1e-7f);
    b = fmaf(b, 0.99999f, 1e-6f);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = t1 - t0;
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
  if (a < 0.f) ticks[2 * blockIdx.x] = 0;  // a stays positive; the test keeps the chain live
}
}  // namespace

constexpr int kClockBlocks = LSH_CLOCK_TICKS_BYTES / 16;

hipError_t launch_clock_spin(unsigned long long* ticks, int blocks, int iters, hipStream_t s) {
  clock_spin_kernel<<<blocks, 256, 0, s>>>(ticks, iters);
  return hipGetLastError();
}
}  // namespace lsh

extern "C" {

const char* lsh_status_string(int status) {
  switch (status) {
    case LSH_OK: return "ok";
    case LSH_ERR_NULL: return "a required pointer is NULL";
    case LSH_ERR_SHAPE: return "invalid shape (negative dimension, D or n_hashes <= 0, L not a multiple of 64 or above 2^24, or int32 index overflow)";
    case LSH_ERR_BUCKETS: return "invalid bucket count (must be 1 or even, at most 4096)";
    case LSH_ERR_UNSUPPORTED: return "unsupported configuration (D and chunk_len must be 64, n_hashes <= 16, dtype f32 or bf16, attend a combination of the LSH_ATTEND_* bits)";
    case LSH_ERR_WORKSPACE: return "workspace missing or too small";
    case LSH_ERR_ALIAS: return "an output overlaps an input";
    case LSH_ERR_HIP: return "HIP launch or event error";
    case LSH_ERR_TOO_LARGE:
      return "one (batch, head) problem needs more than the fixed scratch of the allocation-free forward "
             "(LSH_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int lsh_hash_workspace_bytes(int B, int H, int L, int D, int n_b, int n_h, lsh_dtype dt, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  int st = check_problem(B, H, L, D, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st == LSH_OK && !dtype_ok(dt)) st = LSH_ERR_UNSUPPORTED;
  if (st != LSH_OK) return st;
  *bytes = is_empty(B, H, L) ? 0 : hash_ws(B * H, L, n_b, n_h, dt).total;
  return LSH_OK;
}

int lsh_hash(const void* qk, const void* rot, int32_t* buckets, int B, int H, int L, int D, int n_b, int n_h,
             lsh_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  int st = check_problem(B, H, L, D, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st == LSH_OK && !dtype_ok(dt)) st = LSH_ERR_UNSUPPORTED;
  if (st != LSH_OK) return st;
  if (is_empty(B, H, L)) return LSH_OK;
  if (qk == nullptr || buckets == nullptr || (n_b > 1 && rot == nullptr)) return LSH_ERR_NULL;
  const int BH = B * H;
  const HashWs w = hash_ws(BH, L, n_b, n_h, dt);
  if (n_b > 1 && (ws == nullptr || ws_bytes < w.total)) return LSH_ERR_WORKSPACE;
  const size_t es = elem_size(dt);
  const size_t nb_bytes = (size_t)BH * n_h * L * sizeof(int32_t);
  if (overlaps(buckets, nb_bytes, qk, (size_t)BH * L * kD * es) ||
      overlaps(buckets, nb_bytes, rot, n_b > 1 ? (size_t)n_h * kD * (n_b / 2) * es : 0) ||
      overlaps(buckets, nb_bytes, ws, n_b > 1 ? ws_bytes : 0))
    return LSH_ERR_ALIAS;
  int k = 0;
  return hip_status(enqueue_hash(qk, rot, buckets, nullptr, (char*)ws, w, BH, L, n_b, n_h, dt,
                                 (hipStream_t)stream, nullptr, &k));
}

int lsh_hash_uncertified(const void* ws, size_t ws_bytes, int B, int H, int L, int n_b, int n_h, lsh_dtype dt,
                         int* count, void* stream) {
  if (count == nullptr) return LSH_ERR_NULL;
  int st = check_problem(B, H, L, kD, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st == LSH_OK && !dtype_ok(dt)) st = LSH_ERR_UNSUPPORTED;
  if (st != LSH_OK) return st;
  *count = 0;
  if (is_empty(B, H, L) || n_b == 1) return LSH_OK;
  const HashWs w = hash_ws(B * H, L, n_b, n_h, dt);  // at offset 0 of the hash and forward workspaces
  if (ws == nullptr || ws_bytes < w.total) return LSH_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int v = 0;
  if (hipMemcpyAsync(&v, (const char*)ws + w.fix_count, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return LSH_ERR_HIP;
  *count = v;
  return LSH_OK;
}

int lsh_sort_workspace_bytes(int B, int H, int L, int n_b, int n_h, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  int st = check_problem(B, H, L, kD, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st != LSH_OK) return st;
  *bytes = is_empty(B, H, L) ? 0 : sort_ws_bytes(B * H, L, n_b, n_h);
  return LSH_OK;
}

int lsh_sort(const int32_t* buckets, int32_t* sorted_idx, int32_t* undo_idx, int B, int H, int L, int n_b,
             int n_h, void* ws, size_t ws_bytes, void* stream) {
  int st = check_problem(B, H, L, kD, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st != LSH_OK) return st;
  if (is_empty(B, H, L)) return LSH_OK;
  if (buckets == nullptr || sorted_idx == nullptr || undo_idx == nullptr) return LSH_ERR_NULL;
  const int BH = B * H;
  const size_t need = sort_ws_bytes(BH, L, n_b, n_h);
  if (ws == nullptr || ws_bytes < need) return LSH_ERR_WORKSPACE;
  const size_t nb = (size_t)BH * n_h * L * sizeof(int32_t);
  if (overlaps(sorted_idx, nb, buckets, nb) || overlaps(undo_idx, nb, buckets, nb) ||
      overlaps(sorted_idx, nb, undo_idx, nb) || overlaps(sorted_idx, nb, ws, ws_bytes) ||
      overlaps(undo_idx, nb, ws, ws_bytes) || overlaps(buckets, nb, ws, ws_bytes))
    return LSH_ERR_ALIAS;
  int k = 0;
  return hip_status(enqueue_sort(buckets, sorted_idx, undo_idx, (int*)ws, BH, L, n_b, n_h, (hipStream_t)stream,
                                 nullptr, &k));
}

}  // extern "C"

namespace {

size_t chunk_attn_ws_bytes(int BH, int L, int n_h, int attend) {
  return (attend & LSH_ATTEND_DEDUP) ? align_up((size_t)BH * n_h * L * sizeof(int32_t), kAlign) : 0;
}

}  // namespace

extern "C" {

int lsh_chunk_attn_ex_workspace_bytes(int B, int H, int L, int n_h, int attend, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  const int st = check_problem(B, H, L, kD, n_h);
  if (st != LSH_OK) return st;
  if (!attend_ok(attend)) return LSH_ERR_UNSUPPORTED;
  *bytes = is_empty(B, H, L) ? 0 : chunk_attn_ws_bytes(B * H, L, n_h, attend);
  return LSH_OK;
}

int lsh_chunk_attn_ex(const void* qk, const void* v, const int32_t* sorted_idx, const int32_t* buckets,
                      const int32_t* undo_idx, void* o_sorted, float* lse_sorted, int B, int H, int L, int D,
                      int n_h, int C, int causal, int attend, lsh_dtype dt, void* ws, size_t ws_bytes,
                      void* stream) {
  int st = check_problem(B, H, L, D, n_h);
  if (st != LSH_OK) return st;
  if (C != kChunk) return C <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt) || !attend_ok(attend)) return LSH_ERR_UNSUPPORTED;
  if (is_empty(B, H, L)) return LSH_OK;
  const bool sb = (attend & LSH_ATTEND_SAME_BUCKET) != 0, dd = (attend & LSH_ATTEND_DEDUP) != 0;
  if (qk == nullptr || v == nullptr || sorted_idx == nullptr || o_sorted == nullptr || lse_sorted == nullptr ||
      (sb && buckets == nullptr) || (dd && undo_idx == nullptr))
    return LSH_ERR_NULL;
  const int BH = B * H;
  const size_t need = chunk_attn_ws_bytes(BH, L, n_h, attend);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LSH_ERR_WORKSPACE;
  const size_t es = elem_size(dt);
  const size_t slots = (size_t)BH * n_h * L;
  const size_t in_bytes = (size_t)BH * L * kD * es;
  const size_t o_bytes = slots * kD * es, l_bytes = slots * sizeof(float), i_bytes = slots * sizeof(int32_t);
  const size_t w_bytes = need > 0 ? ws_bytes : 0;
  const void* ins[5] = {qk, v, sorted_idx, sb ? buckets : nullptr, dd ? undo_idx : nullptr};
  const size_t in_n[5] = {in_bytes, in_bytes, i_bytes, i_bytes, i_bytes};
  for (int a = 0; a < 5; ++a)
    if (overlaps(o_sorted, o_bytes, ins[a], in_n[a]) || overlaps(lse_sorted, l_bytes, ins[a], in_n[a]) ||
        overlaps(ws, w_bytes, ins[a], in_n[a]))
      return LSH_ERR_ALIAS;
  if (overlaps(o_sorted, o_bytes, lse_sorted, l_bytes) || overlaps(ws, w_bytes, o_sorted, o_bytes) ||
      overlaps(ws, w_bytes, lse_sorted, l_bytes))
    return LSH_ERR_ALIAS;
  return hip_status(launch_chunk_attn(qk, v, sorted_idx, o_sorted, lse_sorted, nullptr, sb ? buckets : nullptr,
                                      dd ? undo_idx : nullptr, dd ? (int32_t*)ws : nullptr, BH, L, n_h, causal,
                                      attend, dt, (hipStream_t)stream));
}

int lsh_chunk_attn(const void* qk, const void* v, const int32_t* sorted_idx, void* o_sorted, float* lse_sorted,
                   int B, int H, int L, int D, int n_h, int C, int causal, lsh_dtype dt, void* stream) {
  return lsh_chunk_attn_ex(qk, v, sorted_idx, nullptr, nullptr, o_sorted, lse_sorted, B, H, L, D, n_h, C, causal, 0,
                           dt, nullptr, 0, stream);
}

int lsh_unsort_combine(const void* o_sorted, const float* lse_sorted, const int32_t* undo_idx, void* out,
                       float* lse_out, int B, int H, int L, int D, int n_h, lsh_dtype dt, void* stream) {
  int st = check_problem(B, H, L, D, n_h);
  if (st != LSH_OK) return st;
  if (!dtype_ok(dt)) return LSH_ERR_UNSUPPORTED;
  if (is_empty(B, H, L)) return LSH_OK;
  if (o_sorted == nullptr || lse_sorted == nullptr || undo_idx == nullptr || out == nullptr) return LSH_ERR_NULL;
  const int BH = B * H;
  const size_t es = elem_size(dt);
  const size_t slots = (size_t)BH * n_h * L;
  const size_t out_bytes = (size_t)BH * L * kD * es, lo_bytes = (size_t)BH * L * sizeof(float);
  const void* ins[3] = {o_sorted, lse_sorted, undo_idx};
  const size_t in_n[3] = {slots * kD * es, slots * sizeof(float), slots * sizeof(int32_t)};
  for (int a = 0; a < 3; ++a)
    if (overlaps(out, out_bytes, ins[a], in_n[a]) || overlaps(lse_out, lo_bytes, ins[a], in_n[a]))
      return LSH_ERR_ALIAS;
  if (overlaps(out, out_bytes, lse_out, lo_bytes)) return LSH_ERR_ALIAS;
  return hip_status(launch_combine(o_sorted, lse_sorted, undo_idx, out, lse_out, BH, L, n_h, dt,
                                   (hipStream_t)stream));
}

int lsh_fwd_workspace_bytes(int B, int H, int L, int D, int n_b, int n_h, int C, lsh_dtype dt, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  int st = check_problem(B, H, L, D, n_h);
  if (st == LSH_OK) st = check_buckets(n_b, L);
  if (st != LSH_OK) return st;
  if (C != kChunk) return C <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt)) return LSH_ERR_UNSUPPORTED;
  *bytes = is_empty(B, H, L) ? 0 : fwd_ws(B * H, L, n_b, n_h, dt).total;
  return LSH_OK;
}

}  // extern "C"

namespace {

// The launch sequence of the fused forward over BH problems, with every
// intermediate carved from `base` by the layout `w` (fwd_ws of the same BH, L,
// n_b, n_h, dt).  sorted_out / undo_out / lse_sorted_out: all or none.
hipError_t enqueue_forward(const void* qk, const void* v, const void* rot, int n_b, int n_h, int causal, int attend,
                           int BH, int L, lsh_dtype dt, void* out, float* lse_out, int32_t* sorted_out,
                           int32_t* undo_out, float* lse_sorted_out, char* base, const FwdWs& w, hipStream_t s,
                           void* const* stage_events) {
  const bool save = sorted_out != nullptr;
  int32_t* buckets = (int32_t*)(base + w.buckets);
  int32_t* sorted_idx = save ? sorted_out : (int32_t*)(base + w.sorted_idx);
  int32_t* undo_idx = save ? undo_out : (int32_t*)(base + w.undo_idx);
  void* o_sorted = base + w.o_sorted;
  float* lse_sorted = save ? lse_sorted_out : (float*)(base + w.lse_sorted);
  // Per-token attention scales are a by-product of hashing; with one bucket there is
  // no hash pass and the attention computes them itself.
  float2* token_scales = n_b > 1 ? (float2*)(base + w.token_scales) : nullptr;
  int k = 0;
  hipError_t e = hipSuccess;
  e = record_stage(stage_events, 0, s);
  if (e == hipSuccess)
    e = enqueue_hash(qk, rot, buckets, token_scales, base + w.hash_base, w.hash, BH, L, n_b, n_h, dt, s,
                     stage_events, &k);
  if (e == hipSuccess)
    e = enqueue_sort(buckets, sorted_idx, undo_idx, (int*)(base + w.sort_base), BH, L, n_b, n_h, s, stage_events,
                     &k);
  if (e == hipSuccess)
    e = launch_chunk_attn(qk, v, sorted_idx, o_sorted, lse_sorted, token_scales, buckets, undo_idx,
                          (int32_t*)(base + w.tok_rec), BH, L, n_h, causal, attend, dt, s);
  if (e == hipSuccess && stage_events != nullptr) e = record_stage(stage_events, ++k, s);
  if (e == hipSuccess) e = launch_combine(o_sorted, lse_sorted, undo_idx, out, lse_out, BH, L, n_h, dt, s);
  if (e == hipSuccess && stage_events != nullptr) e = record_stage(stage_events, ++k, s);
  return e;
}

// The fused forward; sorted_idx / undo_idx / lse_sorted (all or none) receive
// the state that the backward pass reuses instead of workspace scratch.
int fused_forward(const void* qk, const void* v, const void* rot, int n_buckets, int n_hashes, int chunk_len,
                  int causal, int attend, int B, int H, int L, int D, lsh_dtype dt, void* out, float* lse_out,
                  int32_t* sorted_out, int32_t* undo_out, float* lse_sorted_out, void* ws, size_t ws_bytes,
                  void* stream, void* const* stage_events) {
  int st = check_problem(B, H, L, D, n_hashes);
  if (st == LSH_OK) st = check_buckets(n_buckets, L);
  if (st != LSH_OK) return st;
  if (chunk_len != kChunk) return chunk_len <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt) || !attend_ok(attend)) return LSH_ERR_UNSUPPORTED;
  if (is_empty(B, H, L)) {
    // Nothing to compute; the stage events are still recorded, back to back.
    if (stage_events != nullptr)
      for (int k = 0; k < LSH_FWD_N_EVENTS; ++k)
        if (record_stage(stage_events, k, (hipStream_t)stream) != hipSuccess) return LSH_ERR_HIP;
    return LSH_OK;
  }
  if (qk == nullptr || v == nullptr || out == nullptr || (n_buckets > 1 && rot == nullptr)) return LSH_ERR_NULL;
  const int BH = B * H, n_h = n_hashes, n_b = n_buckets;
  const FwdWs w = fwd_ws(BH, L, n_b, n_h, dt);
  if (ws == nullptr || ws_bytes < w.total) return LSH_ERR_WORKSPACE;
  const size_t es = elem_size(dt);
  const size_t in_bytes = (size_t)BH * L * kD * es;
  const size_t rot_bytes = n_b > 1 ? (size_t)n_h * kD * (n_b / 2) * es : 0;
  const size_t lo_bytes = (size_t)BH * L * sizeof(float);
  const void* ins[4] = {qk, v, rot, ws};
  const size_t in_n[4] = {in_bytes, in_bytes, rot_bytes, ws_bytes};
  for (int a = 0; a < 4; ++a)
    if (overlaps(out, in_bytes, ins[a], in_n[a]) || overlaps(lse_out, lo_bytes, ins[a], in_n[a]))
      return LSH_ERR_ALIAS;
  if (overlaps(out, in_bytes, lse_out, lo_bytes)) return LSH_ERR_ALIAS;
  if (overlaps(ws, ws_bytes, qk, in_bytes) || overlaps(ws, ws_bytes, v, in_bytes) ||
      overlaps(ws, ws_bytes, rot, rot_bytes))
    return LSH_ERR_ALIAS;
  const bool save = sorted_out != nullptr;
  if (save) {
    const size_t slots = (size_t)BH * n_h * L;
    const void* outs[5] = {out, lse_out, sorted_out, undo_out, lse_sorted_out};
    const size_t out_n[5] = {in_bytes, lse_out ? lo_bytes : 0, slots * 4, slots * 4, slots * 4};
    for (int a = 2; a < 5; ++a) {
      for (int b = 0; b < 4; ++b)
        if (overlaps(outs[a], out_n[a], ins[b], in_n[b])) return LSH_ERR_ALIAS;
      for (int b = 0; b < 5; ++b)
        if (b != a && overlaps(outs[a], out_n[a], outs[b], out_n[b])) return LSH_ERR_ALIAS;
    }
  }

  return hip_status(enqueue_forward(qk, v, rot, n_b, n_h, causal, attend, BH, L, dt, out, lse_out, sorted_out,
                                    undo_out, lse_sorted_out, (char*)ws, w, (hipStream_t)stream, stage_events));
}

}  // namespace

extern "C" {

int reformer_lsh_attn_fwd_ex(const void* qk, const void* v, const void* rot, int n_buckets, int n_hashes,
                             int chunk_len, int causal, int attend, int B, int H, int L, int D, lsh_dtype dt,
                             void* out, float* lse_out, void* ws, size_t ws_bytes, void* stream,
                             void* const* stage_events) {
  return fused_forward(qk, v, rot, n_buckets, n_hashes, chunk_len, causal, attend, B, H, L, D, dt, out, lse_out,
                       nullptr, nullptr, nullptr, ws, ws_bytes, stream, stage_events);
}

int reformer_lsh_attn_fwd(const void* qk, const void* v, const void* rot, int n_buckets, int n_hashes, int chunk_len,
                          int causal, int B, int H, int L, int D, lsh_dtype dt, void* out, float* lse_out, void* ws,
                          size_t ws_bytes, void* stream, void* const* stage_events) {
  return fused_forward(qk, v, rot, n_buckets, n_hashes, chunk_len, causal, 0, B, H, L, D, dt, out, lse_out, nullptr,
                       nullptr, nullptr, ws, ws_bytes, stream, stage_events);
}

int reformer_lsh_attn_fwd_train(const void* qk, const void* v, const void* rot, int n_buckets, int n_hashes,
                                int chunk_len, int causal, int B, int H, int L, int D, lsh_dtype dt, void* out,
                                float* lse_out, int32_t* sorted_idx, int32_t* undo_idx, float* lse_sorted, void* ws,
                                size_t ws_bytes, void* stream, void* const* stage_events) {
  const int st = check_problem(B, H, L, D, n_hashes);
  if (st != LSH_OK) return st;
  if (!is_empty(B, H, L) && (sorted_idx == nullptr || undo_idx == nullptr || lse_sorted == nullptr))
    return LSH_ERR_NULL;
  return fused_forward(qk, v, rot, n_buckets, n_hashes, chunk_len, causal, 0, B, H, L, D, dt, out, lse_out,
                       sorted_idx, undo_idx, lse_sorted, ws, ws_bytes, stream, stage_events);
}

}  // extern "C"

// ---- The allocation-free forward: a fixed device scratch in place of the workspace ----
namespace {

// Every device the library runs on holds one copy of this array (allocated when
// the code object is loaded there) until the process ends.  In host code its
// name is only a stand-in: the device address of each device's copy comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[LSH_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first call
// on that device (with the device current) and kept.
hipError_t current_scratch(char** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = (char*)g_scratch_ptr[dev];
  return hipSuccess;
}

// The largest number of (batch, head) problems whose forward workspace fits the
// scratch (0 when one does not).
int noalloc_group(int BH, int L, int n_b, int n_h, lsh_dtype dt) {
  const size_t one = fwd_ws(1, L, n_b, n_h, dt).total;
  if (one > LSH_NOALLOC_SCRATCH_BYTES) return 0;
  int g = (int)(LSH_NOALLOC_SCRATCH_BYTES / one);
  if (g > BH) g = BH;
  while (g > 1 && fwd_ws(g, L, n_b, n_h, dt).total > LSH_NOALLOC_SCRATCH_BYTES) --g;
  return g;
}

}  // namespace

extern "C" {

int reformer_lsh_attn_fwd_noalloc(const void* qk, const void* v, const void* rot, int n_buckets, int n_hashes,
                                  int chunk_len, int causal, int B, int H, int L, int D, lsh_dtype dt, void* out,
                                  float* lse_out, void* stream) {
  int st = check_problem(B, H, L, D, n_hashes);
  if (st == LSH_OK) st = check_buckets(n_buckets, L);
  if (st != LSH_OK) return st;
  if (chunk_len != kChunk) return chunk_len <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt)) return LSH_ERR_UNSUPPORTED;
  if (is_empty(B, H, L)) return LSH_OK;
  if (qk == nullptr || v == nullptr || out == nullptr || (n_buckets > 1 && rot == nullptr)) return LSH_ERR_NULL;
  const int BH = B * H, n_h = n_hashes, n_b = n_buckets;
  const int group = noalloc_group(BH, L, n_b, n_h, dt);
  if (group == 0) return LSH_ERR_TOO_LARGE;
  const size_t es = elem_size(dt);
  const size_t in_bytes = (size_t)BH * L * kD * es;
  const size_t rot_bytes = n_b > 1 ? (size_t)n_h * kD * (n_b / 2) * es : 0;
  const size_t lo_bytes = (size_t)BH * L * sizeof(float);
  const void* ins[3] = {qk, v, rot};
  const size_t in_n[3] = {in_bytes, in_bytes, rot_bytes};
  for (int a = 0; a < 3; ++a)
    if (overlaps(out, in_bytes, ins[a], in_n[a]) || overlaps(lse_out, lo_bytes, ins[a], in_n[a]))
      return LSH_ERR_ALIAS;
  if (overlaps(out, in_bytes, lse_out, lo_bytes)) return LSH_ERR_ALIAS;
  char* base = nullptr;
  hipError_t e = current_scratch(&base);
  if (e != hipSuccess) return LSH_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  // Groups of problems in stream order on the one scratch: each group's kernels
  // finish their reads of it before the next group's first kernel writes it.
  for (int g0 = 0; g0 < BH && e == hipSuccess; g0 += group) {
    const int n = BH - g0 < group ? BH - g0 : group;
    const FwdWs w = fwd_ws(n, L, n_b, n_h, dt);
    const size_t row0 = (size_t)g0 * L;
    e = enqueue_forward((const char*)qk + row0 * kD * es, (const char*)v + row0 * kD * es, rot, n_b, n_h, causal, 0,
                        n, L, dt, (char*)out + row0 * kD * es, lse_out == nullptr ? nullptr : lse_out + row0,
                        nullptr, nullptr, nullptr, base, w, s, nullptr);
  }
  return hip_status(e);
}

int lsh_attn_bwd_workspace_bytes(int B, int H, int L, int D, int n_h, int C, lsh_dtype dt, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  const int st = check_problem(B, H, L, D, n_h);
  if (st != LSH_OK) return st;
  if (C != kChunk) return C <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt)) return LSH_ERR_UNSUPPORTED;
  *bytes = is_empty(B, H, L) ? 0 : bwd_ws(B * H, L, n_h, dt).total;
  return LSH_OK;
}

int lsh_attn_bwd(const void* qk, const void* v, const int32_t* sorted_idx, const int32_t* undo_idx,
                 const float* lse_sorted, const void* out, const void* dout, const float* dlse, void* dqk, void* dv,
                 int B, int H, int L, int D, int n_h, int C, int causal, lsh_dtype dt, void* ws, size_t ws_bytes,
                 void* stream, void* const* stage_events) {
  int st = check_problem(B, H, L, D, n_h);
  if (st != LSH_OK) return st;
  if (C != kChunk) return C <= 0 ? LSH_ERR_SHAPE : LSH_ERR_UNSUPPORTED;
  if (!dtype_ok(dt)) return LSH_ERR_UNSUPPORTED;
  if (is_empty(B, H, L)) {
    if (stage_events != nullptr)
      for (int k = 0; k < LSH_BWD_N_EVENTS; ++k)
        if (record_stage(stage_events, k, (hipStream_t)stream) != hipSuccess) return LSH_ERR_HIP;
    return LSH_OK;
  }
  if (qk == nullptr || v == nullptr || sorted_idx == nullptr || undo_idx == nullptr || lse_sorted == nullptr ||
      out == nullptr || dout == nullptr || dqk == nullptr || dv == nullptr)
    return LSH_ERR_NULL;
  const int BH = B * H;
  const BwdWs w = bwd_ws(BH, L, n_h, dt);
  if (ws == nullptr || ws_bytes < w.total) return LSH_ERR_WORKSPACE;
  const size_t es = elem_size(dt);
  const size_t slots = (size_t)BH * n_h * L;
  const size_t tok_bytes = (size_t)BH * L * kD * es, i_bytes = slots * sizeof(int32_t);
  const void* ins[9] = {qk, v, sorted_idx, undo_idx, lse_sorted, out, dout, dlse, ws};
  const size_t in_n[9] = {tok_bytes, tok_bytes, i_bytes, i_bytes, slots * sizeof(float), tok_bytes, tok_bytes,
                          (size_t)BH * L * sizeof(float), ws_bytes};
  for (int a = 0; a < 9; ++a)
    if (overlaps(dqk, tok_bytes, ins[a], in_n[a]) || overlaps(dv, tok_bytes, ins[a], in_n[a])) return LSH_ERR_ALIAS;
  if (overlaps(dqk, tok_bytes, dv, tok_bytes)) return LSH_ERR_ALIAS;
  for (int a = 0; a < 8; ++a)
    if (overlaps(ws, ws_bytes, ins[a], in_n[a])) return LSH_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  float2* tok_w = (float2*)(base + w.tok_w);
  float2* tok_scale = (float2*)(base + w.tok_scale);
  void* dx_slot = base + w.dx_slot;
  void* dv_slot = base + w.dv_slot;
  int k = 0;
  auto mark = [&](void) -> hipError_t {
    return record_stage(stage_events, k++, s);
  };
  hipError_t e = mark();
  if (e == hipSuccess)
    e = launch_bwd_prep(qk, out, dout, dlse, lse_sorted, undo_idx, tok_w, tok_scale, BH, L, n_h, dt, s);
  if (e == hipSuccess) e = mark();
  if (e == hipSuccess)
    e = launch_attn_bwd(qk, v, dout, sorted_idx, lse_sorted, tok_w, tok_scale, dx_slot, dv_slot, BH, L, n_h, causal,
                        dt, s);
  if (e == hipSuccess) e = mark();
  if (e == hipSuccess) e = launch_bwd_reduce(dx_slot, dv_slot, undo_idx, dqk, dv, BH, L, n_h, dt, s);
  if (e == hipSuccess) e = mark();
  return hip_status(e);
}

int lsh_layer_norm(const void* x, const void* gamma, const void* beta, void* y, int rows, int dim, lsh_dtype dt,
                   void* stream) {
  if (rows < 0 || dim <= 0) return LSH_ERR_SHAPE;
  if (dt != LSH_BF16 || dim % 8 != 0 || dim > 1024) return LSH_ERR_UNSUPPORTED;
  if (rows == 0) return LSH_OK;
  if (x == nullptr || gamma == nullptr || beta == nullptr || y == nullptr) return LSH_ERR_NULL;
  const size_t n = (size_t)rows * dim * 2;
  if (overlaps(y, n, x, n) || overlaps(y, n, gamma, (size_t)dim * 2) || overlaps(y, n, beta, (size_t)dim * 2))
    return LSH_ERR_ALIAS;
  return hip_status(launch_layer_norm(x, gamma, beta, y, rows, dim, (hipStream_t)stream));
}

int lsh_linear(const void* a, int a_layout, const void* w, const void* bias, const void* resid, void* c, int c_layout,
               int M, int N, int K, int L, int heads, int epilogue, lsh_dtype dt, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return LSH_ERR_SHAPE;
  if (dt != LSH_BF16 || N % 128 != 0 || K % 64 != 0) return LSH_ERR_UNSUPPORTED;
  const bool bias_on = (epilogue & LSH_EPI_BIAS) != 0, gelu = (epilogue & LSH_EPI_GELU) != 0,
             resid_on = (epilogue & LSH_EPI_RESID) != 0;
  const int epi = (bias_on ? kEpiBias : 0) | (gelu ? kEpiGelu : 0) | (resid_on ? kEpiResid : 0);
  if ((epilogue & ~(LSH_EPI_BIAS | LSH_EPI_GELU | LSH_EPI_RESID)) != 0 ||
      (epi != 0 && epi != (kEpiBias | kEpiGelu) && epi != kEpiResid && epi != (kEpiBias | kEpiResid)))
    return LSH_ERR_UNSUPPORTED;
  const bool ah = a_layout == LSH_LAYOUT_HEADS, ch = c_layout == LSH_LAYOUT_HEADS;
  if ((a_layout != LSH_LAYOUT_ROWS && !ah) || (c_layout != LSH_LAYOUT_ROWS && !ch) || (ah && ch) || (ch && resid_on))
    return LSH_ERR_UNSUPPORTED;
  if ((ah || ch) && (L <= 0 || heads <= 0 || M % L != 0 || (ah ? K : N) != heads * kD)) return LSH_ERR_SHAPE;
  if (M == 0) return LSH_OK;
  if (a == nullptr || w == nullptr || c == nullptr || (bias_on && bias == nullptr) || (resid_on && resid == nullptr))
    return LSH_ERR_NULL;
  const size_t na = (size_t)M * K * 2, nc = (size_t)M * N * 2, nw = (size_t)N * K * 2;
  if (overlaps(c, nc, a, na) || overlaps(c, nc, w, nw) || overlaps(c, nc, bias_on ? bias : nullptr, (size_t)N * 2) ||
      overlaps(c, nc, resid_on ? resid : nullptr, nc))
    return LSH_ERR_ALIAS;
  return hip_status(launch_gemm(a, ah ? kLayoutHeads : kLayoutRows, w, bias, resid, c, ch ? kLayoutHeads : kLayoutRows,
                                M, N, K, ah || ch ? L : 1, ah || ch ? heads : 1, epi, (hipStream_t)stream));
}

int reformer_block_workspace_bytes(int B, int L, int heads, int n_buckets, int n_hashes, int chunk_len,
                                   int chunk_rows, lsh_dtype dt, size_t* bytes) {
  if (bytes == nullptr) return LSH_ERR_NULL;
  const int st = check_block(B, L, heads, n_buckets, n_hashes, chunk_len, chunk_rows, dt);
  if (st != LSH_OK) return st;
  *bytes = is_empty(B, heads, L) ? 0 : block_ws(B, L, heads, n_buckets, n_hashes, chunk_rows).total;
  return LSH_OK;
}

int reformer_block_fwd(const void* x1, const void* x2, const void* rot, const void* const* params, int B, int L,
                       int heads, int n_buckets, int n_hashes, int chunk_len, int causal, int chunk_rows,
                       lsh_dtype dt, void* y1, void* y2, void* ws, size_t ws_bytes, void* stream,
                       void* const* stage_events) {
  const int st = check_block(B, L, heads, n_buckets, n_hashes, chunk_len, chunk_rows, dt);
  if (st != LSH_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (is_empty(B, heads, L)) {
    if (stage_events != nullptr)
      for (int k = 0; k < LSH_BLOCK_N_EVENTS; ++k)
        if (record_stage(stage_events, k, s) != hipSuccess) return LSH_ERR_HIP;
    return LSH_OK;
  }
  if (x1 == nullptr || x2 == nullptr || params == nullptr || y1 == nullptr || y2 == nullptr ||
      (n_buckets > 1 && rot == nullptr))
    return LSH_ERR_NULL;
  for (int k = 0; k < LSH_BLOCK_N_PARAMS; ++k)
    if (params[k] == nullptr) return LSH_ERR_NULL;
  const BlockWs w = block_ws(B, L, heads, n_buckets, n_hashes, chunk_rows);
  if (ws == nullptr || ws_bytes < w.total) return LSH_ERR_WORKSPACE;
  const int M = B * L, dim = heads * kD;
  const size_t act = (size_t)M * dim * 2;
  const size_t pn[LSH_BLOCK_N_PARAMS] = {(size_t)dim * 2, (size_t)dim * 2, (size_t)dim * dim * 2,
                                         (size_t)dim * dim * 2, (size_t)dim * dim * 2, (size_t)dim * 2,
                                         (size_t)dim * 2, (size_t)4 * dim * dim * 2, (size_t)4 * dim * 2,
                                         (size_t)4 * dim * dim * 2, (size_t)dim * 2};
  const size_t rot_bytes = n_buckets > 1 ? (size_t)n_hashes * kD * (n_buckets / 2) * 2 : 0;
  const void* outs[2] = {y1, y2};
  for (int o = 0; o < 2; ++o) {
    if (overlaps(outs[o], act, x1, act) || overlaps(outs[o], act, x2, act) ||
        overlaps(outs[o], act, rot, rot_bytes) || overlaps(outs[o], act, ws, ws_bytes))
      return LSH_ERR_ALIAS;
    for (int k = 0; k < LSH_BLOCK_N_PARAMS; ++k)
      if (overlaps(outs[o], act, params[k], pn[k])) return LSH_ERR_ALIAS;
  }
  if (overlaps(y1, act, y2, act) || overlaps(ws, ws_bytes, x1, act) || overlaps(ws, ws_bytes, x2, act) ||
      overlaps(ws, ws_bytes, rot, rot_bytes))
    return LSH_ERR_ALIAS;
  for (int k = 0; k < LSH_BLOCK_N_PARAMS; ++k)
    if (overlaps(ws, ws_bytes, params[k], pn[k])) return LSH_ERR_ALIAS;

  char* base = (char*)ws;
  void* h1 = base + w.h1;
  void* qk = base + w.qk;
  void* v = base + w.v;
  void* att = base + w.att;
  void* h2 = base + w.h2;
  void* hid = base + w.hid;
  int k = 0;
  auto mark = [&](void) -> hipError_t {
    return record_stage(stage_events, k++, s);
  };
  const void* const* p = params;
  hipError_t e = mark();
  // y1 = x1 + W_o . attention(LN1(x2) W_qk^T, LN1(x2) W_v^T)
  if (e == hipSuccess) e = launch_layer_norm(x2, p[LSH_BLOCK_LN1_G], p[LSH_BLOCK_LN1_B], h1, M, dim, s);
  if (e == hipSuccess) e = mark();
  if (e == hipSuccess)
    e = launch_gemm(h1, kLayoutRows, p[LSH_BLOCK_W_QK], nullptr, nullptr, qk, kLayoutHeads, M, dim, dim, L, heads, 0, s);
  if (e == hipSuccess)
    e = launch_gemm(h1, kLayoutRows, p[LSH_BLOCK_W_V], nullptr, nullptr, v, kLayoutHeads, M, dim, dim, L, heads, 0, s);
  if (e == hipSuccess) e = mark();
  if (e != hipSuccess) return hip_status(e);
  const int ast = fused_forward(qk, v, rot, n_buckets, n_hashes, chunk_len, causal, 0, B, heads, L, kD, dt, att,
                                nullptr, nullptr, nullptr, nullptr, base + w.attn_base, w.attn.total, stream, nullptr);
  if (ast != LSH_OK) return ast;
  e = mark();
  if (e == hipSuccess)
    e = launch_gemm(att, kLayoutHeads, p[LSH_BLOCK_W_O], nullptr, x1, y1, kLayoutRows, M, dim, dim, L, heads,
                    kEpiResid, s);
  if (e == hipSuccess) e = mark();
  // y2 = x2 + W2 . GELU(W1 . LN2(y1) + b1) + b2, the hidden activation a chunk of rows at a time
  if (e == hipSuccess) e = launch_layer_norm(y1, p[LSH_BLOCK_LN2_G], p[LSH_BLOCK_LN2_B], h2, M, dim, s);
  if (e == hipSuccess) e = mark();
  const int rows = chunk_rows > 0 && chunk_rows < M ? chunk_rows : M;
  for (int r0 = 0; r0 < M && e == hipSuccess; r0 += rows) {
    const int m = M - r0 < rows ? M - r0 : rows;
    const size_t off = (size_t)r0 * dim * 2;
    e = launch_gemm((const char*)h2 + off, kLayoutRows, p[LSH_BLOCK_W1], p[LSH_BLOCK_B1], nullptr, hid, kLayoutRows,
                    m, 4 * dim, dim, L, heads, kEpiBias | kEpiGelu, s);
    if (e == hipSuccess)
      e = launch_gemm(hid, kLayoutRows, p[LSH_BLOCK_W2], p[LSH_BLOCK_B2], (const char*)x2 + off, (char*)y2 + off,
                      kLayoutRows, m, dim, 4 * dim, L, heads, kEpiBias | kEpiResid, s);
  }
  if (e == hipSuccess) e = mark();
  return hip_status(e);
}

int lsh_event_create(void** event) {
  if (event == nullptr) return LSH_ERR_NULL;
  // Timing only: a record without the system-scope fence writes no caches
  // back for the host, so it delays the next kernel by about one microsecond
  // instead of a few.
  hipEvent_t e;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return LSH_ERR_HIP;
  *event = (void*)e;
  return LSH_OK;
}

int lsh_event_destroy(void* event) {
  if (event == nullptr) return LSH_ERR_NULL;
  return hip_status(hipEventDestroy((hipEvent_t)event));
}

int lsh_event_record(void* event, void* stream) {
  if (event == nullptr) return LSH_ERR_NULL;
  return hip_status(hipEventRecord((hipEvent_t)event, (hipStream_t)stream));
}

int lsh_event_elapsed_ms(void* start, void* end, float* ms) {
  if (start == nullptr || end == nullptr || ms == nullptr) return LSH_ERR_NULL;
  if (hipEventSynchronize((hipEvent_t)end) != hipSuccess) return LSH_ERR_HIP;
  return hip_status(hipEventElapsedTime(ms, (hipEvent_t)start, (hipEvent_t)end));
}

int lsh_measure_clock(void* ticks, int spin_us, double* mhz, void* stream) {
  if (ticks == nullptr || mhz == nullptr) return LSH_ERR_NULL;
  if (spin_us < 1 || spin_us > 100000) return LSH_ERR_SHAPE;
  int dev = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz <= 0)
    return LSH_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  // about 24 iterations per microsecond at 8 waves per SIMD
  if (lsh::launch_clock_spin((unsigned long long*)ticks, lsh::kClockBlocks, 24 * spin_us, s) != hipSuccess)
    return LSH_ERR_HIP;
  std::vector<unsigned long long> h(2 * lsh::kClockBlocks);
  if (hipMemcpyAsync(h.data(), ticks, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return LSH_ERR_HIP;
  double cycles = 0.0, real = 0.0;
  for (int b = 0; b < lsh::kClockBlocks; ++b) {
    cycles += (double)h[2 * b];
    real += (double)h[2 * b + 1];
  }
  *mhz = real > 0.0 ? cycles / real * (double)wall_khz / 1e3 : 0.0;
  return LSH_OK;
}

}  // extern "C"
