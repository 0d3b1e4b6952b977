// Internal declarations shared by the HIP kernels and the C-ABI host layer.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
// (layer, KV head) slices per workgroup, one wave per slice: the re-RoPE
// scatter launches n_sel * ceil(L*H_kv / kScatterSlices) workgroups of
// kScatterThreads; the working-set update n_new * ceil(L*H_kv / kWorksetChunk)
// workgroups of 64 * kWorksetSlices threads, each wave taking every
// kWorksetSlices-th slice of the workgroup's chunk
constexpr int kScatterSlices = 16;
constexpr int kScatterThreads = 64 * kScatterSlices;
constexpr int kWorksetSlices = 8;
constexpr int kWorksetChunk = 8;

// bf16 is the top half of a binary32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
// float32 -> bf16 through gfx950's conversion instruction (v_cvt_pk_bf16_f32):
// round to nearest even, subnormals kept, a NaN stays a NaN.  One instruction
// converts a pair, where rounding by hand took about nine.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Merge two (max, sum-of-exp2(x - max)) pairs.  Empty pairs are (-inf, 0).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
  m = mn;
}

inline unsigned ceil_div(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Buffer accesses through a resource over [base, base + bytes): a scalar base
// and a 32-bit per-lane offset, bounds-checked by the hardware (writes past
// `bytes` are dropped).  `base` must be wave-uniform.  aux is the cache
// policy operand: 0 = default, kBufSc1 = write through to memory, kBufNt =
// non-temporal.
constexpr int kBufWord3 = 0x00020000;   // resource word 3 for raw (untyped) access on gfx9
constexpr int kBufSc1 = 16;
constexpr int kBufNt = 2;              // non-temporal: data read or written once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufWord3);
}
// A 16-byte store takes its whole offset in the per-lane (vector) offset with
// a zero scalar offset.  gfx9 needs a wait state between a store of more than
// 8 bytes and a VALU write of its data registers; the compiler inserts it only
// when the scalar offset is the constant 0.  With an SGPR scalar offset, a
// store that reads its data late (under heavy memory traffic) could store a
// register the next instruction had already rewritten.
template <int AUX = 0>
__device__ __forceinline__ void buf_store16(u32x4 v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, AUX);
}
// 4- and 1-byte forms; a load past `bytes` returns 0.
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store1(uint8_t v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, byte_off, 0, 0);
}

}  // namespace kvs

// Launchers (host side).  Each returns the launch status; arguments are
// already validated by the C-ABI layer.
hipError_t kvs_launch_qmem(const void* q, int dtype, int L, int H_q, int S, int D, float decay,
                           int first_turn, float* M, hipStream_t st);

// slots == nullptr: K is dense [L, H_kv, N, D]; otherwise K is the token-major
// pool [L, pool_size, H_kv, D] read through the slot map slots[N].
hipError_t kvs_launch_rule(const void* K, int dtype, const int64_t* slots, int64_t pool_size,
                           const float* M, int L, int H_q, int H_kv, int D, int64_t N, int64_t pi,
                           int64_t q_s, int64_t q_e, float* rule, void* ws, hipStream_t st);
size_t kvs_rule_ws_bytes(int L, int H_q, int H_kv, int64_t N);
// Sets the fold's bounded wait (polls; < 0: every chunk takes the spill path);
// returns the previous value.
int64_t kvs_rule_fold_spin(int64_t polls);

// slot_out != nullptr: the emit also writes slot_out[j] = kept ? slot_in[j] : dead_slot.
hipError_t kvs_launch_topk(const float* score, int64_t n, int64_t f0b, int64_t f0e, int64_t f1b,
                           int64_t f1e, int64_t n_forced, int64_t c_star, uint8_t* keep_mask,
                           int32_t* keep_idx, int64_t* n_kept, void* ws, hipStream_t st,
                           const int64_t* slot_in, int64_t dead_slot, int64_t* slot_out);
size_t kvs_topk_ws_bytes(int64_t n);
// Same selection with the multi-workgroup state in the library's own static
// device array (no workspace); n <= kvs_topk_noalloc_max_n().
int64_t kvs_topk_noalloc_max_n();
hipError_t kvs_launch_topk_noalloc(const float* score, int64_t n, int64_t f0b, int64_t f0e, int64_t f1b,
                                   int64_t f1e, int64_t n_forced, int64_t c_star, uint8_t* keep_mask,
                                   int32_t* keep_idx, int64_t* n_kept, hipStream_t st);

hipError_t kvs_launch_slotmap(const int64_t* in, const uint8_t* mask, int64_t N, int64_t dead,
                              int64_t* out, hipStream_t st);

hipError_t kvs_launch_meank_build(const void* K, int L, int H_kv, int D, int64_t N, int k_is_rope,
                                  int64_t pos0, double theta, void* raw_out, void* index,
                                  hipStream_t st);

hipError_t kvs_launch_meank_append(const void* chunk, int L, int H_kv, int D, int64_t t0, int64_t n_new,
                                   int64_t pos0, double theta, void* stage, int64_t cap, void* index,
                                   hipStream_t st);

hipError_t kvs_launch_meank_score(const void* Q, const void* index, int L, int H_q, int H_kv, int D,
                                  int64_t Mq, int64_t nB, int64_t c0, int64_t c1, float* R,
                                  void* ws, hipStream_t st);
size_t kvs_meank_ws_bytes(int L, int H_q, int H_kv, int64_t Mq, int64_t nB);

hipError_t kvs_launch_rerope(const void* k_src, const void* v_src, int64_t src_tokens,
                             const int32_t* src_block, const int32_t* page_table, int64_t n_sel,
                             int L, int H_kv, int D, int64_t pos_base, double theta, void* k_pool,
                             void* v_pool, int64_t pool_pages, int32_t* err_flag, hipStream_t st);

size_t kvs_workset_ws_bytes(int64_t pool_pages);
hipError_t kvs_launch_workset(const void* k_src, const void* v_src, int64_t src_tokens,
                              const int32_t* prev_blocks, const int32_t* prev_pages, int64_t n_prev,
                              const int32_t* new_blocks, int64_t n_new, int L, int H_kv, int D,
                              int64_t pos_base, double theta, void* k_pool, void* v_pool,
                              int64_t pool_pages, int32_t* pages_out, int32_t* old_rank_out,
                              int32_t* outgoing_out, int64_t* counts, int32_t* err_flag, void* ws,
                              hipStream_t st);

size_t kvs_window_ws_bytes(int L, int H_q, int H_kv, int64_t W, int64_t N);
hipError_t kvs_launch_window(const void* K, const void* Qw, int L, int H_q, int H_kv, int D, int64_t W, int64_t N,
                             int64_t pi, int64_t q_s, int64_t q_e, float* score, void* ws, hipStream_t st);
