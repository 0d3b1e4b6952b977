// Differential working-set update of the execution view (KVMEM, section
// "Engineering and cost: tiered movement, page-table aliasing and
// position-consistent reconstruction"): only blocks the step selects that the
// page pool does not already hold are materialised again.
//
// W_t (new_blocks) and G_{t-1} (prev_blocks, with their pages) are ascending
// block ids; a block's compact index is its rank.  Classes:
//   retained  (in both)      keeps its page; if its rank moved, its K is rebuilt
//                            from raw K (the reconstruction authority) at the new
//                            positions, like an incoming block; V is untouched.
//                            This moves the same bytes as rotating the pool's copy
//                            by the position delta, without rounding the block to
//                            bf16 once more per move (no drift over many steps).
//   incoming  (W_t only)     takes a free page -- one no retained block holds,
//                            free pages in ascending order to incoming blocks in
//                            ascending rank -- and is written like the re-RoPE
//                            scatter: raw K rotated to its compact positions, V copied.
//   outgoing  (G_{t-1} only) releases its page.
// Two kernels: workset_diff (one workgroup: binary searches, block-wide
// scans, the new page table) and workset_apply (one workgroup per selected
// block and chunk of slices: re-RoPE from raw K, V copy for incoming blocks,
// or nothing for a block retained at the same rank).
#include "rope_table.h"

using namespace kvs;

namespace {

constexpr int kBlk = 32;
constexpr int kThreads = 1024;

// Exclusive prefix sum over the workgroup; *total gets the sum.  All threads call it.
__device__ __forceinline__ int block_scan(int x, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    const int v = sh[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

// First index i in [0, n) with a[i] >= key (a ascending), n if none.
__device__ __forceinline__ int64_t lower_bound(const int32_t* a, int64_t n, int32_t key) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void workset_diff(
    const int32_t* __restrict__ prev_blocks, const int32_t* __restrict__ prev_pages, int64_t n_prev,
    const int32_t* __restrict__ new_blocks, int64_t n_new, int64_t src_blocks, int64_t pool_pages,
    int32_t* __restrict__ held, int32_t* __restrict__ pages_out, int32_t* __restrict__ old_rank_out,
    int32_t* __restrict__ outgoing_out, int64_t* __restrict__ counts, int32_t* __restrict__ err_flag) {
  __shared__ int sh[kThreads / 64];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  for (int64_t p = tid; p < pool_pages; p += kThreads) held[p] = 0;
  __syncthreads();

  // Ranks, input checks, and the pages retained blocks hold.
  for (int64_t r = tid; r < n_new; r += kThreads) {
    const int32_t b = new_blocks[r];
    bool bad = b < 0 || b >= src_blocks || (r > 0 && new_blocks[r - 1] >= b);
    const int64_t i = lower_bound(prev_blocks, n_prev, b);
    int32_t rank = -1;
    if (i < n_prev && prev_blocks[i] == b) {
      rank = (int32_t)i;
      const int32_t p = prev_pages[i];
      if (p < 0 || p >= pool_pages) bad = true;
      else if (atomicAdd(&held[p], 1) != 0) bad = true;      // two retained blocks on one page
    }
    old_rank_out[r] = rank;
    if (bad) s_bad = 1;
  }
  for (int64_t i = tid; i < n_prev; i += kThreads)
    if (i > 0 && prev_blocks[i - 1] >= prev_blocks[i]) s_bad = 1;
  __syncthreads();

  // Outgoing pages, in G_{t-1} order.
  int n_out = 0;
  for (int64_t i0 = 0; i0 < n_prev; i0 += kThreads) {
    const int64_t i = i0 + tid;
    int out = 0;
    if (i < n_prev) {
      const int64_t j = lower_bound(new_blocks, n_new, prev_blocks[i]);
      out = !(j < n_new && new_blocks[j] == prev_blocks[i]);
    }
    int tot;
    const int pre = block_scan(out, sh, &tot);
    if (out) outgoing_out[n_out + pre] = prev_pages[i];
    n_out += tot;
  }

  // Free pages (held by no retained block) in ascending order, written over `held`
  // from the front: entry k of the free list lands at held[k] <= its own page, so
  // a pass only overwrites entries an earlier pass has already read.
  int n_free = 0;
  for (int64_t p0 = 0; p0 < pool_pages; p0 += kThreads) {
    const int64_t p = p0 + tid;
    const int f = p < pool_pages ? held[p] == 0 : 0;
    int tot;
    const int pre = block_scan(f, sh, &tot);       // its barriers order the reads above before the writes below
    if (f) held[n_free + pre] = (int32_t)p;
    n_free += tot;
    __syncthreads();
  }

  // The new page table: retained blocks keep their page, incoming take free pages in rank order.
  int n_inc = 0;
  for (int64_t r0 = 0; r0 < n_new; r0 += kThreads) {
    const int64_t r = r0 + tid;
    const int inc = r < n_new ? old_rank_out[r] < 0 : 0;
    int tot;
    const int pre = block_scan(inc, sh, &tot);
    if (r < n_new) {
      const int32_t rank = old_rank_out[r];
      int32_t page = -1;
      if (rank >= 0) page = prev_pages[rank];
      else if (n_inc + pre < n_free) page = held[n_inc + pre];
      pages_out[r] = s_bad ? -1 : page;
    }
    n_inc += tot;
  }
  if (tid == 0) {
    counts[0] = n_new - n_inc;
    counts[1] = n_inc;
    counts[2] = n_out;
    if ((s_bad || n_inc > n_free) && err_flag) *err_flag = 1;
  }
}

// One workgroup per (selected block, chunk of kWorksetSlices slices), chunks
// fastest, one slice per wave of a 512-thread workgroup: short-lived
// workgroups stream faster than one workgroup per block over every slice, and
// a wave with one slice never waits for its stores before further loads.
// Same-process A/B at meank-256k: 5.09 ms against 5.12 ms with two slices per
// wave of 256 threads.  The scatter's 16-slice, 1024-thread shape was 4% slower
// here: most workgroups belong to blocks retained in place, which exit at
// once, and large workgroups cost more to launch and retire.  At meank-1m
// (512 slices, half the selected blocks moved, half incoming) that shape is
// 4% faster (6.43 against 6.70 ms), and 32- or 64-slice chunks over 8 waves
// 2-3%; the 8-slice shape stays for the sizes where blocks stay in place.
template <int D, bool WITH_V>
__global__ __launch_bounds__(64 * kWorksetSlices, 2) void workset_apply(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, int64_t src_tokens,
    const int32_t* __restrict__ new_blocks, const int32_t* __restrict__ pages,
    const int32_t* __restrict__ old_rank, int LG, int64_t pos_base, double log2_theta,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool, int64_t pool_pages) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  __shared__ float2 tab[kBlk][D / 2];
  const int nch = (LG + kWorksetChunk - 1) / kWorksetChunk;
  const int r = blockIdx.x / nch, chunk = blockIdx.x % nch;
  const int32_t rank = old_rank[r];
  const int64_t page = pages[r];
  if (page < 0 || page >= pool_pages || rank == r) return;      // rejected input, or retained in place
  const bool moved = rank >= 0;                                 // retained, rank changed: V stays
  const int64_t sb = new_blocks[r];
  build_rope_table<D>(tab, pos_base + (int64_t)kBlk * r, log2_theta);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  // one 32 x D block of one slice through buffer resources (wave-uniform base,
  // the lane's byte offset; each load's row group is a scalar offset, each
  // store's is added to the lane's offset)
  constexpr int kBlkBytes = kBlk * D * 2, kGroupBytes = RPL * D * 2;
  const int lane_off = (rr * D + cl * 8) * 2;
  const int64_t pool_tokens = pool_pages * kBlk;
  const int lg_end = min(LG, (chunk + 1) * kWorksetChunk);
  for (int lg = chunk * kWorksetChunk + wave; lg < lg_end; lg += kWorksetSlices) {
    const size_t d0 = ((size_t)lg * pool_tokens + (size_t)page * kBlk) * D;
    const size_t s0 = ((size_t)lg * src_tokens + (size_t)sb * kBlk) * D;
    const auto kin = buf_rsrc(k_src + s0, kBlkBytes);
    const auto kd = buf_rsrc(k_pool + d0, kBlkBytes);
    asm volatile("" ::: "memory");   // table reads stay in the loop (held across it they cost 128 VGPRs)
    u32x4 w[LOADS], vv[LOADS];
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) w[ld] = __builtin_amdgcn_raw_buffer_load_b128(kin, lane_off, ld * kGroupBytes, 0);
    if constexpr (WITH_V) {
      if (!moved) {
        const auto vs = buf_rsrc(v_src + s0, kBlkBytes);
#pragma unroll
        for (int ld = 0; ld < LOADS; ++ld) vv[ld] = __builtin_amdgcn_raw_buffer_load_b128(vs, lane_off, ld * kGroupBytes, 0);
      }
    }
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      float x[8];
      unpack8(w[ld], x);
      rotate8<D>(x, tab[ld * RPL + rr], cl, +1);
      buf_store16(pack8(x), kd, lane_off + ld * kGroupBytes);   // whole offset per lane (see buf_store16)
    }
    if constexpr (WITH_V) {
      if (!moved) {
        const auto vd = buf_rsrc(v_pool + d0, kBlkBytes);
#pragma unroll
        for (int ld = 0; ld < LOADS; ++ld) buf_store16(vv[ld], vd, lane_off + ld * kGroupBytes);
      }
    }
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t kvs_workset_ws_bytes(int64_t pool_pages) { return align256((size_t)pool_pages * 4); }

hipError_t kvs_launch_workset(const void* k_src, const void* v_src, int64_t src_tokens,
                              const int32_t* prev_blocks, const int32_t* prev_pages, int64_t n_prev,
                              const int32_t* new_blocks, int64_t n_new, int L, int H_kv, int D,
                              int64_t pos_base, double theta, void* k_pool, void* v_pool,
                              int64_t pool_pages, int32_t* pages_out, int32_t* old_rank_out,
                              int32_t* outgoing_out, int64_t* counts, int32_t* err_flag, void* ws,
                              hipStream_t st) {
  hipLaunchKernelGGL(workset_diff, dim3(1), dim3(kThreads), 0, st, prev_blocks, prev_pages, n_prev,
                     new_blocks, n_new, src_tokens / kBlk, pool_pages, static_cast<int32_t*>(ws), pages_out,
                     old_rank_out, outgoing_out, counts, err_flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_new == 0) return e;
  const int LG = L * H_kv;
  const double l2t = __builtin_log2(theta);
  const uint16_t* ks = static_cast<const uint16_t*>(k_src);
  const uint16_t* vs = static_cast<const uint16_t*>(v_src);
  uint16_t* kp = static_cast<uint16_t*>(k_pool);
  uint16_t* vp = static_cast<uint16_t*>(v_pool);
  const dim3 grid((unsigned)(n_new * ceil_div(LG, kWorksetChunk))), block(64 * kWorksetSlices);
#define KVS_APPLY(DD, WV)                                                                          \
  hipLaunchKernelGGL((workset_apply<DD, WV>), grid, block, 0, st, ks, vs, src_tokens, new_blocks, \
                     pages_out, old_rank_out, LG, pos_base, l2t, kp, vp, pool_pages)
  if (D == 128) {
    if (vs) KVS_APPLY(128, true);
    else KVS_APPLY(128, false);
  } else {
    if (vs) KVS_APPLY(64, true);
    else KVS_APPLY(64, false);
  }
#undef KVS_APPLY
  return hipGetLastError();
}
