// Re-RoPE scatter into the execution view (KVMEM, section "Engineering and
// cost: tiered movement, page-table aliasing and position-consistent
// reconstruction"): for each selected block r, raw K is rotated to the
// compact positions pos_base + 32r + t and written to physical page
// page_table[r]; V is copied unchanged.
//
// HBM-bound (read K and V once, write them once).  A workgroup owns one
// selected block for every (layer, KV head): it builds the block's 32 x D/2
// rotation table once in LDS (float64 angles) and streams the L*H_kv 32-row
// blocks of K and V through it with 16-byte coalesced loads and stores.
// Out-of-range block ids or pages skip the block and raise err_flag instead of
// touching memory outside the buffers.
#include "rope_table.h"

using namespace kvs;

namespace {

constexpr int kBlk = 32;

template <int D>
__global__ __launch_bounds__(256) void rerope_scatter_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int64_t src_tokens,
    const int32_t* __restrict__ src_block, const int32_t* __restrict__ page_table, int LG,
    int64_t pos_base, double log2_theta, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, int64_t pool_pages, int32_t* __restrict__ err_flag) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  __shared__ float2 tab[kBlk][D / 2];
  const int r = blockIdx.x;
  const int64_t sb = src_block[r];
  const int64_t dst = page_table ? (int64_t)page_table[r] : (int64_t)r;
  if (sb < 0 || (sb + 1) * kBlk > src_tokens || dst < 0 || dst >= pool_pages) {
    if (threadIdx.x == 0 && err_flag) *err_flag = 1;
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  build_rope_table<D>(tab, pos_base + (int64_t)kBlk * r, log2_theta);
  __syncthreads();
  const int64_t pool_tokens = pool_pages * kBlk;
  for (int lg = wave; lg < LG; lg += 4) {
    const size_t s0 = ((size_t)lg * src_tokens + (size_t)sb * kBlk) * D + cl * 8;
    const size_t d0 = ((size_t)lg * pool_tokens + (size_t)dst * kBlk) * D + cl * 8;
    u32x4 w[LOADS], vv[LOADS];
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const size_t off = (size_t)(ld * RPL + rr) * D;
      w[ld] = *reinterpret_cast<const u32x4*>(k_src + s0 + off);
      if (v_src) vv[ld] = *reinterpret_cast<const u32x4*>(v_src + s0 + off);
    }
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int t = ld * RPL + rr;
      float x[8];
      unpack8(w[ld], x);
      rotate8<D>(x, tab[t], cl, +1);
      const size_t off = (size_t)t * D;
      *reinterpret_cast<u32x4*>(k_pool + d0 + off) = pack8(x);
      if (v_src) *reinterpret_cast<u32x4*>(v_pool + d0 + off) = vv[ld];
    }
  }
}

}  // namespace

hipError_t kvs_launch_rerope(const void* k_src, const void* v_src, int64_t src_tokens,
                             const int32_t* src_block, const int32_t* page_table, int64_t n_sel,
                             int L, int H_kv, int D, int64_t pos_base, double theta, void* k_pool,
                             void* v_pool, int64_t pool_pages, int32_t* err_flag, hipStream_t st) {
  if (n_sel == 0) return hipSuccess;
  const int LG = L * H_kv;
  const double l2t = __builtin_log2(theta);
  dim3 grid((unsigned)n_sel), block(256);
  const uint16_t* ks = static_cast<const uint16_t*>(k_src);
  const uint16_t* vs = static_cast<const uint16_t*>(v_src);
  uint16_t* kp = static_cast<uint16_t*>(k_pool);
  uint16_t* vp = static_cast<uint16_t*>(v_pool);
  if (D == 128)
    hipLaunchKernelGGL(rerope_scatter_kernel<128>, grid, block, 0, st, ks, vs, src_tokens, src_block,
                       page_table, LG, pos_base, l2t, kp, vp, pool_pages, err_flag);
  else
    hipLaunchKernelGGL(rerope_scatter_kernel<64>, grid, block, 0, st, ks, vs, src_tokens, src_block,
                       page_table, LG, pos_base, l2t, kp, vp, pool_pages, err_flag);
  return hipGetLastError();
}
