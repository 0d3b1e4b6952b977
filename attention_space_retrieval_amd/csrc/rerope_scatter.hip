// Re-RoPE scatter into the execution view (KVMEM, section "Engineering and
// cost: tiered movement, page-table aliasing and position-consistent
// reconstruction"): for each selected block r, raw K is rotated to the
// compact positions pos_base + 32r + t and written to physical page
// page_table[r]; V is copied unchanged.
//
// HBM-bound (read K and V once, write them once).  A workgroup owns one
// selected block for a chunk of 16 (layer, KV head) slices: it builds the
// block's 32 x D/2 rotation table in LDS (float64 angles), then each of its
// 16 waves streams one slice's 32-row block of K through it with 16-byte
// coalesced loads and stores.  The grid runs the chunks of a block fastest.
// One slice per wave matters: a wave that loops over two slices waits for its
// first slice's stores before it can use its second slice's loads (gfx9 counts
// both on one counter).  Same-process A/B for 2048 blocks over 512 slices:
// 6.50 ms with 8 slices per workgroup at two per wave, 6.46 ms at one per wave,
// 6.42 ms with 16 slices at one per wave (4 slices: 6.55 ms).
// Out-of-range block ids or pages skip the block and raise err_flag instead
// of touching memory outside the buffers.
#include "rope_table.h"

using namespace kvs;

namespace {

constexpr int kBlk = 32;
constexpr int kLgChunk = kScatterSlices;   // (layer, KV head) slices per workgroup, one per wave

template <int D>
__global__ __launch_bounds__(kScatterThreads, 1) void rerope_scatter_kernel(
    const uint16_t* __restrict__ k_src, int64_t src_tokens, const int32_t* __restrict__ src_block,
    const int32_t* __restrict__ page_table, int LG, int64_t pos_base, double log2_theta,
    uint16_t* __restrict__ k_pool, int64_t pool_pages, int32_t* __restrict__ err_flag) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  __shared__ float2 tab[kBlk][D / 2];
  // workgroup -> (selected block r, chunk of slices), chunks fastest: the
  // workgroups in flight cover every slice of a few neighbouring blocks
  const int nch = (LG + kLgChunk - 1) / kLgChunk;
  const int r = blockIdx.x / nch, chunk = blockIdx.x % nch;
  const int64_t sb = src_block[r];
  const int64_t dst = page_table ? (int64_t)page_table[r] : (int64_t)r;
  if (sb < 0 || (sb + 1) * kBlk > src_tokens || dst < 0 || dst >= pool_pages) {
    if (threadIdx.x == 0 && err_flag) *err_flag = 1;
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  build_rope_table<D>(tab, pos_base + (int64_t)kBlk * r, log2_theta);
  __syncthreads();
  // one 32 x D block of one slice through buffer resources: a wave-uniform
  // base and the lane's byte offset; each load's row group is a scalar offset,
  // each store's is added to the lane's offset
  constexpr int kBlkBytes = kBlk * D * 2, kGroupBytes = RPL * D * 2;
  const int lane_off = (rr * D + cl * 8) * 2;
  const int64_t pool_tokens = pool_pages * kBlk;
  const int lg_end = min(LG, (chunk + 1) * kLgChunk);
  for (int lg = chunk * kLgChunk + wave; lg < lg_end; lg += kScatterThreads / 64) {
    const size_t s0 = ((size_t)lg * src_tokens + (size_t)sb * kBlk) * D;
    const size_t d0 = ((size_t)lg * pool_tokens + (size_t)dst * kBlk) * D;
    const auto ks = buf_rsrc(k_src + s0, kBlkBytes), kd = buf_rsrc(k_pool + d0, kBlkBytes);
    // the lane's 64 table entries are the same for every slice, but held in
    // registers across the loop they would cost 128 VGPRs: re-read them from
    // LDS per slice (a memory clobber keeps the reads inside the loop)
    asm volatile("" ::: "memory");
    u32x4 w[LOADS];
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) w[ld] = __builtin_amdgcn_raw_buffer_load_b128(ks, lane_off, ld * kGroupBytes, 0);
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      float x[8];
      unpack8(w[ld], x);
      rotate8<D>(x, tab[ld * RPL + rr], cl, +1);
      buf_store16(pack8(x), kd, lane_off + ld * kGroupBytes);   // whole offset per lane (see buf_store16)
    }
  }
}

// V carries no position: a plain copy, one 16-byte load and one store per
// thread, 4 KB per workgroup (half a block at D = 128, a whole one at D = 64).
// The grid runs the pieces of one block fastest, then the blocks (x), then
// the slices (y).  Short workgroups that load once and store once move these
// scattered pieces faster than workgroups that loop over slices, whose every
// later load also waits for the earlier stores (one counter tracks both).
template <int D>
__global__ __launch_bounds__(256) void v_scatter_kernel(const uint16_t* __restrict__ v_src, int64_t src_tokens,
                                                        const int32_t* __restrict__ src_block,
                                                        const int32_t* __restrict__ page_table,
                                                        uint16_t* __restrict__ v_pool, int64_t pool_pages) {
  constexpr int kPieceBytes = 256 * 16, kPieces = kBlk * D * 2 / kPieceBytes;
  const int piece = (int)(blockIdx.x % kPieces);
  const int64_t r = blockIdx.x / kPieces, lg = blockIdx.y;
  const int64_t sb = src_block[r];
  const int64_t dst = page_table ? (int64_t)page_table[r] : r;
  if (sb < 0 || (sb + 1) * kBlk > src_tokens || dst < 0 || dst >= pool_pages) return;   // K's kernel flags it
  const size_t s0 = ((size_t)lg * src_tokens + (size_t)sb * kBlk) * D;
  const size_t d0 = ((size_t)lg * pool_pages * kBlk + (size_t)dst * kBlk) * D;
  const auto vs = buf_rsrc(v_src + s0, kBlk * D * 2), vd = buf_rsrc(v_pool + d0, kBlk * D * 2);
  const int off = piece * kPieceBytes + threadIdx.x * 16;
  buf_store16(__builtin_amdgcn_raw_buffer_load_b128(vs, off, 0, 0), vd, off);
}

}  // namespace

hipError_t kvs_launch_rerope(const void* k_src, const void* v_src, int64_t src_tokens,
                             const int32_t* src_block, const int32_t* page_table, int64_t n_sel,
                             int L, int H_kv, int D, int64_t pos_base, double theta, void* k_pool,
                             void* v_pool, int64_t pool_pages, int32_t* err_flag, hipStream_t st) {
  if (n_sel == 0) return hipSuccess;
  const int LG = L * H_kv;
  const double l2t = __builtin_log2(theta);
  dim3 grid((unsigned)(n_sel * ceil_div(LG, kLgChunk))), block(kScatterThreads);
  const uint16_t* ks = static_cast<const uint16_t*>(k_src);
  const uint16_t* vs = static_cast<const uint16_t*>(v_src);
  uint16_t* kp = static_cast<uint16_t*>(k_pool);
  uint16_t* vp = static_cast<uint16_t*>(v_pool);
  if (D == 128)
    hipLaunchKernelGGL(rerope_scatter_kernel<128>, grid, block, 0, st, ks, src_tokens, src_block, page_table, LG,
                       pos_base, l2t, kp, pool_pages, err_flag);
  else
    hipLaunchKernelGGL(rerope_scatter_kernel<64>, grid, block, 0, st, ks, src_tokens, src_block, page_table, LG,
                       pos_base, l2t, kp, pool_pages, err_flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !vs) return e;
  const dim3 vgrid((unsigned)(n_sel * (kBlk * D * 2 / 4096)), (unsigned)LG);
  if (D == 128)
    hipLaunchKernelGGL(v_scatter_kernel<128>, vgrid, dim3(256), 0, st, vs, src_tokens, src_block, page_table, vp,
                       pool_pages);
  else
    hipLaunchKernelGGL(v_scatter_kernel<64>, vgrid, dim3(256), 0, st, vs, src_tokens, src_block, page_table, vp,
                       pool_pages);
  return hipGetLastError();
}
