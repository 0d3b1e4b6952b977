// C-ABI entry points: host-side validation, then stream-ordered launches.
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the stream.
#include <cmath>
#include <cstdint>
#include <limits>

#include "../../include/kvs.h"
#include "kvs_internal.h"

namespace {

constexpr int64_t kMaxIndex = std::numeric_limits<int32_t>::max();

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Elements of an [a, b, c, d] tensor, or -1 on overflow.
int64_t numel4(int64_t a, int64_t b, int64_t c, int64_t d) {
  int64_t x, y, z;
  if (!mul_ok(a, b, &x) || !mul_ok(x, c, &y) || !mul_ok(y, d, &z)) return -1;
  return z <= (std::numeric_limits<int64_t>::max() >> 2) ? z : -1;
}

bool head_dim_ok(int32_t D) { return D == 64 || D == 128; }

// A 1-D launch of 256-thread workgroups covers at most 2^32 - 1 work-items.
bool grid_ok(int64_t workgroups) { return workgroups >= 0 && workgroups < ((int64_t)1 << 24); }
// The Mean-K / window engine addresses one streamed operand (index blocks,
// query rows or keys of one (layer, KV head)) through a buffer resource with
// 32-bit byte offsets, 256 bytes a row, a few tiles past the end included.
constexpr int64_t kMaxStreamRows = ((int64_t)1 << 23) - 128;
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The kernels move 16-byte vectors: tensor bases (and workspaces) must be 16-byte aligned.
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kvs_status hip_status(hipError_t e) { return e == hipSuccess ? KVS_OK : KVS_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

void clip_range(int64_t n, int64_t& b, int64_t& e) {
  b = b < 0 ? 0 : (b > n ? n : b);
  e = e < b ? b : (e > n ? n : e);
}

// Argument checks shared by the two top-k entry points; clips the forced
// ranges and gives |F| and C*.
kvs_status topk_args(const float* score, int64_t n, int64_t& f0_begin, int64_t& f0_end, int64_t& f1_begin,
                     int64_t& f1_end, int64_t C, const uint8_t* keep_mask, const int32_t* keep_idx,
                     const int64_t* n_kept, int64_t* n_forced, int64_t* c_star) {
  if (!n_kept || (n > 0 && (!score || !keep_mask || !keep_idx))) return KVS_ERR_ARG;
  if (n < 0 || C < 0 || f0_end < f0_begin || f1_end < f1_begin) return KVS_ERR_ARG;
  if (n > kMaxIndex) return KVS_ERR_SHAPE;
  clip_range(n, f0_begin, f0_end);
  clip_range(n, f1_begin, f1_end);
  const int64_t lo = f0_begin > f1_begin ? f0_begin : f1_begin;
  const int64_t hi = f0_end < f1_end ? f0_end : f1_end;
  const int64_t overlap = hi > lo ? hi - lo : 0;
  *n_forced = (f0_end - f0_begin) + (f1_end - f1_begin) - overlap;
  *c_star = C > *n_forced ? C - *n_forced : 0;
  return KVS_OK;
}

}  // namespace

extern "C" {

const char* kvs_status_string(kvs_status s) {
  switch (s) {
    case KVS_OK: return "ok";
    case KVS_ERR_ARG: return "invalid argument";
    case KVS_ERR_SHAPE: return "inconsistent or oversized shape";
    case KVS_ERR_DTYPE: return "unsupported dtype";
    case KVS_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVS_ERR_WORKSPACE: return "workspace missing or too small";
    case KVS_ERR_HIP: return "HIP launch failed";
    case KVS_ERR_LIMIT: return "size above the fixed limit of a no-allocation entry point";
    default: return "unknown status";
  }
}

int32_t kvs_version(void) { return 100; }

kvs_status kvs_qmem_update(const void* q_span, int32_t q_dtype, int32_t L, int32_t H_q, int32_t S,
                           int32_t D, float lambda, int32_t first_turn, float* M, void* stream) {
  if (!q_span || !M || !a16(q_span)) return KVS_ERR_ARG;
  if (q_dtype != KVS_F32 && q_dtype != KVS_BF16) return KVS_ERR_DTYPE;
  if (L < 1 || H_q < 1 || S < 1 || std::isnan(lambda) || lambda < 0.f) return KVS_ERR_ARG;
  if (!head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (numel4(L, H_q, S, D) < 0) return KVS_ERR_SHAPE;
  const float decay = std::isinf(lambda) ? 0.f : std::exp(-lambda);
  return hip_status(kvs_launch_qmem(q_span, q_dtype, L, H_q, S, D, decay, first_turn ? 1 : 0, M,
                                    as_stream(stream)));
}

size_t kvs_rule_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t N) {
  if (L < 1 || H_q < 1 || H_kv < 1 || N < 0 || N > kMaxIndex) return 0;
  return kvs_rule_ws_bytes(L, H_q, H_kv, N);
}

kvs_status kvs_rule_score(const void* K, int32_t k_dtype, const float* M, int32_t L, int32_t H_q,
                          int32_t H_kv, int32_t D, int64_t N, int64_t pi, int64_t q_s, int64_t q_e,
                          float* rule, void* ws, size_t ws_bytes, void* stream) {
  if (!M || (N > 0 && (!K || !rule)) || !a16(K)) return KVS_ERR_ARG;   // K and rule are empty when N = 0
  if (k_dtype != KVS_F32 && k_dtype != KVS_BF16) return KVS_ERR_DTYPE;
  if (L < 1 || H_q < 1 || H_kv < 1 || N < 0 || pi < 0 || q_s < 0 || q_e < q_s) return KVS_ERR_ARG;
  if (H_q % H_kv != 0 || N > kMaxIndex || numel4(L, H_kv, N, D) < 0 ||
      numel4(L, H_q, N, 1) < 0 || (int64_t)L * H_kv > 65535)
    return KVS_ERR_SHAPE;
  if (!head_dim_ok(D) || H_q / H_kv > 16) return KVS_ERR_UNSUPPORTED;
  if (N == 0) return KVS_OK;
  const size_t need = kvs_rule_ws_bytes(L, H_q, H_kv, N);
  if (!ws || ws_bytes < need || !a16(ws)) return KVS_ERR_WORKSPACE;
  pi = pi > N ? N : pi;
  int64_t s = q_s, e = q_e;
  clip_range(N, s, e);
  return hip_status(kvs_launch_rule(K, k_dtype, nullptr, 0, M, L, H_q, H_kv, D, N, pi, s, e, rule, ws,
                                    as_stream(stream)));
}

kvs_status kvs_rule_score_paged(const void* K_pool, int32_t k_dtype, const int64_t* slots,
                                int64_t pool_size, const float* M, int32_t L, int32_t H_q,
                                int32_t H_kv, int32_t D, int64_t N, int64_t pi, int64_t q_s,
                                int64_t q_e, float* rule, void* ws, size_t ws_bytes, void* stream) {
  if (!K_pool || !M || (N > 0 && !rule) || !a16(K_pool)) return KVS_ERR_ARG;
  if (k_dtype != KVS_F32 && k_dtype != KVS_BF16) return KVS_ERR_DTYPE;
  if (L < 1 || H_q < 1 || H_kv < 1 || N < 0 || pool_size < 1 || pi < 0 || q_s < 0 || q_e < q_s)
    return KVS_ERR_ARG;
  if (N > 0 && !slots) return KVS_ERR_ARG;
  if (H_q % H_kv != 0 || N > kMaxIndex || pool_size > kMaxIndex || numel4(L, pool_size, H_kv, D) < 0 ||
      numel4(L, H_q, N, 1) < 0 || (int64_t)L * H_kv > 65535)
    return KVS_ERR_SHAPE;
  if (!head_dim_ok(D) || H_q / H_kv > 16) return KVS_ERR_UNSUPPORTED;
  if (N == 0) return KVS_OK;
  const size_t need = kvs_rule_ws_bytes(L, H_q, H_kv, N);
  if (!ws || ws_bytes < need || !a16(ws)) return KVS_ERR_WORKSPACE;
  pi = pi > N ? N : pi;
  int64_t s = q_s, e = q_e;
  clip_range(N, s, e);
  return hip_status(kvs_launch_rule(K_pool, k_dtype, slots, pool_size, M, L, H_q, H_kv, D, N, pi, s, e,
                                    rule, ws, as_stream(stream)));
}

int64_t kvs_rule_score_wait_limit(int64_t polls) { return kvs_rule_fold_spin(polls); }

size_t kvs_topk_workspace(int64_t n) {
  if (n < 0 || n > kMaxIndex) return 0;
  return kvs_topk_ws_bytes(n);
}

kvs_status kvs_topk_select(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                           int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                           int32_t* keep_idx, int64_t* n_kept, void* ws, size_t ws_bytes,
                           void* stream) {
  int64_t n_forced = 0, c_star = 0;
  const kvs_status a = topk_args(score, n, f0_begin, f0_end, f1_begin, f1_end, C, keep_mask, keep_idx,
                                 n_kept, &n_forced, &c_star);
  if (a != KVS_OK) return a;
  const size_t need = kvs_topk_ws_bytes(n);
  if (need && ws && ws_bytes < need) return KVS_ERR_WORKSPACE;   // no workspace: one-workgroup path
  if (need && ((uintptr_t)ws & 3)) return KVS_ERR_ARG;
  if (!need) ws = nullptr;
  return hip_status(kvs_launch_topk(score, n, f0_begin, f0_end, f1_begin, f1_end, n_forced, c_star,
                                    keep_mask, keep_idx, n_kept, ws, as_stream(stream), nullptr, 0, nullptr));
}

kvs_status kvs_topk_select_redirect(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                                    int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                                    int32_t* keep_idx, int64_t* n_kept, const int64_t* slot_in,
                                    int64_t dead_slot, int64_t* slot_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  int64_t n_forced = 0, c_star = 0;
  const kvs_status a = topk_args(score, n, f0_begin, f0_end, f1_begin, f1_end, C, keep_mask, keep_idx,
                                 n_kept, &n_forced, &c_star);
  if (a != KVS_OK) return a;
  if (n > 0 && (!slot_in || !slot_out)) return KVS_ERR_ARG;
  const size_t need = kvs_topk_ws_bytes(n);
  if (need && ws && ws_bytes < need) return KVS_ERR_WORKSPACE;
  if (need && ((uintptr_t)ws & 3)) return KVS_ERR_ARG;
  if (!need) ws = nullptr;
  return hip_status(kvs_launch_topk(score, n, f0_begin, f0_end, f1_begin, f1_end, n_forced, c_star,
                                    keep_mask, keep_idx, n_kept, ws, as_stream(stream), slot_in, dead_slot,
                                    n > 0 ? slot_out : nullptr));
}

int64_t kvs_topk_noalloc_max(void) { return kvs_topk_noalloc_max_n(); }

kvs_status kvs_topk_select_noalloc(const float* score, int64_t n, int64_t f0_begin, int64_t f0_end,
                                   int64_t f1_begin, int64_t f1_end, int64_t C, uint8_t* keep_mask,
                                   int32_t* keep_idx, int64_t* n_kept, void* stream) {
  int64_t n_forced = 0, c_star = 0;
  const kvs_status a = topk_args(score, n, f0_begin, f0_end, f1_begin, f1_end, C, keep_mask, keep_idx,
                                 n_kept, &n_forced, &c_star);
  if (a != KVS_OK) return a;
  if (n > kvs_topk_noalloc_max_n()) return KVS_ERR_LIMIT;
  return hip_status(kvs_launch_topk_noalloc(score, n, f0_begin, f0_end, f1_begin, f1_end, n_forced, c_star,
                                            keep_mask, keep_idx, n_kept, as_stream(stream)));
}

kvs_status kvs_slotmap_redirect(const int64_t* slot_in, const uint8_t* keep_mask, int64_t N,
                                int64_t dead_slot, int64_t* slot_out, void* stream) {
  if (N < 0 || (N > 0 && (!slot_in || !keep_mask || !slot_out))) return KVS_ERR_ARG;
  return hip_status(kvs_launch_slotmap(slot_in, keep_mask, N, dead_slot, slot_out,
                                       as_stream(stream)));
}

kvs_status kvs_meank_build(const void* K, int32_t L, int32_t H_kv, int32_t D, int64_t N,
                           int32_t block, int32_t k_is_rope, int64_t pos0, double theta,
                           void* raw_k_out, void* index, void* stream) {
  if (!K || !index || !a16(K) || !a16(index) || !a16(raw_k_out)) return KVS_ERR_ARG;
  if (L < 1 || H_kv < 1 || N < 0 || pos0 < 0) return KVS_ERR_ARG;
  if (k_is_rope && !(std::isfinite(theta) && theta > 0.0)) return KVS_ERR_ARG;
  if (block != 32 || !head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (numel4(L, H_kv, N, D) < 0 || (N + 31) / 32 > kMaxIndex || !grid_ok(cdiv(N, 32)) ||
      (k_is_rope && raw_k_out && !grid_ok(cdiv(N, 32) * cdiv((int64_t)L * H_kv, kvs::kScatterSlices))))
    return KVS_ERR_SHAPE;
  return hip_status(kvs_launch_meank_build(K, L, H_kv, D, N, k_is_rope ? 1 : 0, pos0, theta,
                                           k_is_rope ? raw_k_out : nullptr, index,
                                           as_stream(stream)));
}

kvs_status kvs_meank_append(const void* k_chunk, int32_t L, int32_t H_kv, int32_t D, int64_t t0,
                            int64_t n_new, int64_t pos0, double theta, void* raw_stage, int64_t cap,
                            void* index, void* stream) {
  if (L < 1 || H_kv < 1 || t0 < 0 || n_new < 0 || cap < 0 || pos0 < 0) return KVS_ERR_ARG;
  if (!(std::isfinite(theta) && theta > 0.0)) return KVS_ERR_ARG;
  if (!head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (t0 > cap || n_new > cap - t0 || numel4(L, H_kv, cap, D) < 0 || (cap + 31) / 32 > kMaxIndex ||
      (int64_t)L * H_kv > 65535 * 32 || !grid_ok(cdiv(cap, 32)))
    return KVS_ERR_SHAPE;
  if (n_new == 0) return KVS_OK;
  if (!k_chunk || !raw_stage || !index || !a16(k_chunk) || !a16(raw_stage) || !a16(index))
    return KVS_ERR_ARG;
  return hip_status(kvs_launch_meank_append(k_chunk, L, H_kv, D, t0, n_new, pos0, theta, raw_stage, cap,
                                            index, as_stream(stream)));
}

size_t kvs_meank_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t Mq, int64_t nB) {
  if (L < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || Mq < 0 || nB < 0) return 0;
  return kvs_meank_ws_bytes(L, H_q, H_kv, Mq, nB);
}

kvs_status kvs_meank_score(const void* Q, const void* index, int32_t L, int32_t H_q, int32_t H_kv,
                           int32_t D, int64_t Mq, int64_t nB, int64_t n_sink, int64_t n_recent,
                           float* R, void* ws, size_t ws_bytes, void* stream) {
  if (L < 1 || H_q < 1 || H_kv < 1 || Mq < 0 || nB < 0 || n_sink < 0 || n_recent < 0)
    return KVS_ERR_ARG;
  // Q is empty when Mq = 0 (every R_b is then 0), the index and R when nB = 0
  if ((Mq > 0 && !Q) || (nB > 0 && (!index || !R)) || !a16(Q) || !a16(index)) return KVS_ERR_ARG;
  if (H_q % H_kv != 0 || numel4(L, H_q, Mq, D) < 0 || numel4(L, H_kv, nB, D) < 0 ||
      (int64_t)L * H_kv > 65535 || nB > kMaxIndex)
    return KVS_ERR_SHAPE;
  if (!head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (!grid_ok(cdiv((int64_t)(H_q / H_kv) * Mq, 256) * L * H_kv) || !grid_ok(cdiv(nB, 256) * L * H_kv) ||
      nB > kMaxStreamRows || (int64_t)(H_q / H_kv) * Mq > kMaxStreamRows)
    return KVS_ERR_SHAPE;
  if (nB == 0) return KVS_OK;
  const size_t need = kvs_meank_ws_bytes(L, H_q, H_kv, Mq, nB);
  if (!ws || ws_bytes < need || !a16(ws)) return KVS_ERR_WORKSPACE;
  const int64_t c0 = n_sink < nB ? n_sink : nB;
  int64_t c1 = nB - n_recent;
  if (c1 < c0) c1 = c0;
  return hip_status(kvs_launch_meank_score(Q, index, L, H_q, H_kv, D, Mq, nB, c0, c1, R, ws,
                                           as_stream(stream)));
}

kvs_status kvs_rerope_scatter(const void* k_src, const void* v_src, int64_t src_tokens,
                              const int32_t* src_block, const int32_t* page_table, int64_t n_sel,
                              int32_t L, int32_t H_kv, int32_t D, int32_t block, int64_t pos_base,
                              double theta, void* k_pool, void* v_pool, int64_t pool_pages,
                              int32_t* err_flag, void* stream) {
  if (!k_src || !k_pool || (n_sel > 0 && !src_block)) return KVS_ERR_ARG;
  if (!a16(k_src) || !a16(v_src) || !a16(k_pool) || !a16(v_pool)) return KVS_ERR_ARG;
  if ((v_src == nullptr) != (v_pool == nullptr)) return KVS_ERR_ARG;
  if (L < 1 || H_kv < 1 || src_tokens < 0 || n_sel < 0 || pool_pages < 0 || pos_base < 0)
    return KVS_ERR_ARG;
  if (!(std::isfinite(theta) && theta > 0.0)) return KVS_ERR_ARG;
  if (block != 32 || !head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (src_tokens % block != 0 || numel4(L, H_kv, src_tokens, D) < 0 ||
      numel4(L, H_kv, pool_pages, (int64_t)block * D) < 0 ||
      !grid_ok(2 * n_sel) || !grid_ok(n_sel * cdiv((int64_t)L * H_kv, kvs::kScatterSlices)) ||
      (int64_t)L * H_kv > 65535)
    return KVS_ERR_SHAPE;
  return hip_status(kvs_launch_rerope(k_src, v_src, src_tokens, src_block, page_table, n_sel, L,
                                      H_kv, D, pos_base, theta, k_pool, v_pool, pool_pages,
                                      err_flag, as_stream(stream)));
}

size_t kvs_window_score_workspace(int32_t L, int32_t H_q, int32_t H_kv, int64_t W, int64_t N) {
  if (L < 1 || H_q < 1 || H_kv < 1 || H_q % H_kv || W < 0 || N < 0 || N > kMaxIndex) return 0;
  return kvs_window_ws_bytes(L, H_q, H_kv, W, N);
}

kvs_status kvs_window_score(const void* K, const void* Qw, int32_t L, int32_t H_q, int32_t H_kv,
                            int32_t D, int64_t N, int64_t W, int64_t pi, int64_t q_s, int64_t q_e,
                            float* score, void* ws, size_t ws_bytes, void* stream) {
  if (L < 1 || H_q < 1 || H_kv < 1 || N < 0 || W < 1 || pi < 0 || q_s < 0 || q_e < q_s) return KVS_ERR_ARG;
  if (!Qw || (N > 0 && (!K || !score)) || !a16(K) || !a16(Qw)) return KVS_ERR_ARG;   // K, score empty when N = 0
  if (H_q % H_kv != 0 || N > kMaxIndex || numel4(L, H_kv, N, D) < 0 || numel4(L, H_q, W, D) < 0 ||
      (int64_t)L * H_kv > 65535 || (int64_t)(H_q / H_kv) * W > (int64_t)1 << 24 ||
      !grid_ok(cdiv((int64_t)(H_q / H_kv) * W, 256) * L * H_kv) || !grid_ok(cdiv(N, 256) * L * H_kv) ||
      N > kMaxStreamRows || (int64_t)(H_q / H_kv) * W > kMaxStreamRows)
    return KVS_ERR_SHAPE;
  if (!head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (N == 0) return KVS_OK;
  const size_t need = kvs_window_ws_bytes(L, H_q, H_kv, W, N);
  if (!ws || ws_bytes < need || !a16(ws)) return KVS_ERR_WORKSPACE;
  return hip_status(kvs_launch_window(K, Qw, L, H_q, H_kv, D, W, N, pi, q_s, q_e, score, ws, as_stream(stream)));
}

size_t kvs_working_set_workspace(int64_t pool_pages) {
  if (pool_pages < 0 || pool_pages > kMaxIndex) return 0;
  return kvs_workset_ws_bytes(pool_pages);
}

kvs_status kvs_working_set_update(const void* k_src, const void* v_src, int64_t src_tokens,
                                  const int32_t* prev_blocks, const int32_t* prev_pages, int64_t n_prev,
                                  const int32_t* new_blocks, int64_t n_new, int32_t L, int32_t H_kv,
                                  int32_t D, int32_t block, int64_t pos_base, double theta,
                                  void* k_pool, void* v_pool, int64_t pool_pages, int32_t* pages_out,
                                  int32_t* old_rank_out, int32_t* outgoing_pages_out,
                                  int64_t* counts_out, int32_t* err_flag, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (L < 1 || H_kv < 1 || src_tokens < 0 || n_prev < 0 || n_new < 0 || pool_pages < 0 || pos_base < 0)
    return KVS_ERR_ARG;
  if (!(std::isfinite(theta) && theta > 0.0)) return KVS_ERR_ARG;
  if (!k_src || !k_pool || !counts_out || (n_new > 0 && (!new_blocks || !pages_out || !old_rank_out)) ||
      (n_prev > 0 && (!prev_blocks || !prev_pages || !outgoing_pages_out)))
    return KVS_ERR_ARG;
  if (!a16(k_src) || !a16(v_src) || !a16(k_pool) || !a16(v_pool)) return KVS_ERR_ARG;
  if ((v_src == nullptr) != (v_pool == nullptr)) return KVS_ERR_ARG;
  if (block != 32 || !head_dim_ok(D)) return KVS_ERR_UNSUPPORTED;
  if (src_tokens % block != 0 || numel4(L, H_kv, src_tokens, D) < 0 ||
      numel4(L, H_kv, pool_pages, (int64_t)block * D) < 0 || pool_pages > kMaxIndex ||
      n_new > pool_pages || n_prev > pool_pages || !grid_ok(n_new) ||
      !grid_ok(n_new * cdiv((int64_t)L * H_kv, kvs::kWorksetChunk)))
    return KVS_ERR_SHAPE;
  const size_t need = kvs_workset_ws_bytes(pool_pages);
  if (need > 0 && (!ws || ws_bytes < need || !a16(ws))) return KVS_ERR_WORKSPACE;
  return hip_status(kvs_launch_workset(k_src, v_src, src_tokens, prev_blocks, prev_pages, n_prev,
                                       new_blocks, n_new, L, H_kv, D, pos_base, theta, k_pool, v_pool,
                                       pool_pages, pages_out, old_rank_out, outgoing_pages_out,
                                       counts_out, err_flag, ws, as_stream(stream)));
}

}  // extern "C"
