// Mean-K index build (KVMEM, section "Design and trade-offs: step-level
// attention trigger and Mean-K model-native retrieval"): one mean of
// position-free K per 32-token block, per layer and KV head.
//
// HBM-bound stream of K (read once) plus a 1/32-size write.  Sums are float32
// in a fixed order and the mean is rounded to bf16 nearest-even.
//
// De-RoPE mode: the keys carry RoPE at positions pos0 + i.  A workgroup builds
// its token block's 32 x D/2 rotation table once in LDS (float64 angles) and
// takes its (layer, KV head) slices through it: all of them, 4 waves in turn,
// when only the index is written; 16 of them, one per wave, when the RoPE-free
// keys are written out too.
#include "rope_table.h"

using namespace kvs;

namespace {

constexpr int kBlk = 32;
// Sums start from -0 and absent rows read as -0: -0 is the additive identity
// (x + -0 = x for every x, -0 included), so each sum is exactly the float32
// sum of the block's rows, and a block of -0 keys averages to -0.
constexpr float kNegZero = -0.0f;
constexpr u32x4 kNegZeroRows = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};

// The index rows are a thin write stream inside a saturated read stream.
// Written through to memory at once (the sc1 cache policy) they cost about
// half as much as ordinary stores, which sit dirty in L2 until the read stream
// evicts them: ~0.55 ms less on a 34 GB build.  The store is a 16-byte buffer
// store over the row's 256 bytes (the resource also bounds it in hardware);
// two 8-byte write-through stores were ~0.3 ms slower.  `row` must be
// wave-uniform: it becomes the scalar buffer resource.
template <int D>
__device__ __forceinline__ void store_row_through(uint16_t* row, int cl, u32x4 v) {
  buf_store16<kBufSc1>(v, buf_rsrc(row, D * 2), cl * 16);
}

// Raw mode.  One wavefront per block: each load instruction moves 64*8/D
// whole contiguous rows (16-byte non-temporal loads, since K is read once), a
// lane adds the rows it loaded for its 16-byte column chunk, and the row groups
// are folded with a fixed xor butterfly.  The grid has one wavefront per block
// (up to 2^24 blocks; beyond that waves stride over the rest): with many
// short-lived workgroups in flight the HBM stream runs faster than with a
// persistent grid.
template <int D>
__global__ __launch_bounds__(256) void meank_build_raw(const uint16_t* __restrict__ K, int64_t N,
                                                       int64_t nB, int64_t total_blocks,
                                                       uint16_t* __restrict__ index) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  const int lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // keeps gb wave-uniform
  for (int64_t gb = (int64_t)blockIdx.x * 4 + wave; gb < total_blocks; gb += (int64_t)gridDim.x * 4) {
    const int64_t lg = gb / nB, b = gb - lg * nB;
    const int nb = (int)min<int64_t>(kBlk, N - b * kBlk);
    const uint16_t* src = K + ((size_t)lg * N + (size_t)b * kBlk + rr) * D + cl * 8;
    u32x4 w[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      w[i] = i * RPL + rr < nb ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)i * RPL * D))
                               : kNegZeroRows;
    float acc[8] = {kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero};
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      float x[8];
      unpack8(w[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    if (rr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = nb == kBlk ? acc[e] * (1.f / kBlk) : acc[e] / (float)nb;
      store_row_through<D>(index + (size_t)gb * D, cl, pack8(acc));
    }
  }
}

// De-RoPE mode, one workgroup per token block over every (layer, KV head)
// slice: its 4 waves take the slices in turn through the block's rotation
// table.  The launcher uses it when only the index is written: with no stores
// of their own in the loop, long-lived waves keep the loads flowing, and one
// table serves all slices (5.9-6.7 ms at meank-256k by box, 4-6% below the
// layout below in the same process).  Taking the unused raw_out store out of
// this kernel made it 4% slower, so it keeps its general form.
template <int D>
__global__ __launch_bounds__(256) void meank_build_derope(const uint16_t* __restrict__ K, int64_t N,
                                                          int64_t nB, int LG, int64_t pos0,
                                                          double log2_theta,
                                                          uint16_t* __restrict__ raw_out,
                                                          uint16_t* __restrict__ index) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  __shared__ float2 tab[kBlk][D / 2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  const int64_t b = blockIdx.x;
  const int64_t t0 = b * kBlk;
  const int nb = (int)min<int64_t>(kBlk, N - t0);
  build_rope_table<D>(tab, pos0 + t0, log2_theta);
  __syncthreads();
  for (int lg = wave; lg < LG; lg += 4) {
    const size_t row0 = (size_t)lg * N + t0;
    const uint16_t* src = K + row0 * D + cl * 8;
    u32x4 w[LOADS];
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int t = ld * RPL + rr;
      w[ld] = t < nb ? *reinterpret_cast<const u32x4*>(src + (size_t)t * D) : kNegZeroRows;
    }
    float acc[8] = {kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero};
#pragma unroll
    for (int ld = 0; ld < LOADS; ++ld) {
      const int t = ld * RPL + rr;
      float x[8];
      unpack8(w[ld], x);
      rotate8<D>(x, tab[t < nb ? t : 0], cl, -1);
      if (t < nb) {
        if (raw_out) *reinterpret_cast<u32x4*>(raw_out + (row0 + t) * D + cl * 8) = pack8(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
      }
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    if (rr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = nb == kBlk ? acc[e] * (1.f / kBlk) : acc[e] / (float)nb;
      *reinterpret_cast<u32x4*>(index + ((size_t)lg * nB + b) * D + cl * 8) = pack8(acc);
    }
  }
}

// De-RoPE mode with the RoPE-free keys written out.  A workgroup owns one
// token block for a chunk of kScatterSlices (layer, KV head) slices, one slice
// per wave, the layout of the re-RoPE scatter: it builds the block's 32 x D/2
// rotation table once in LDS (float64 angles), then each wave streams its
// slice's block through it with 16-byte loads and stores through buffer
// resources (rows past the end read as zero and their stores are dropped) and
// writes the block's mean.  The grid runs the chunks of a block fastest.  A
// wave that loops over slices waits for its stores before the next slice's
// loads (one counter for both): 13.13 ms at meank-256k, against 13.6 ms for
// the layout above with the keys written out.
template <int D>
__global__ __launch_bounds__(kScatterThreads, 1) void meank_build_derope_out(const uint16_t* __restrict__ K, int64_t N,
                                                                       int64_t nB, int LG, int64_t pos0,
                                                                       double log2_theta,
                                                                       uint16_t* __restrict__ raw_out,
                                                                       uint16_t* __restrict__ index) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  constexpr int kGroupBytes = RPL * D * 2;
  __shared__ float2 tab[kBlk][D / 2];
  const int nch = (LG + kScatterSlices - 1) / kScatterSlices;
  const int64_t b = blockIdx.x / nch;
  const int chunk = blockIdx.x % nch;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  const int64_t t0 = b * kBlk;
  const int nb = (int)min<int64_t>(kBlk, N - t0);
  build_rope_table<D>(tab, pos0 + t0, log2_theta);
  __syncthreads();
  const int lg = chunk * kScatterSlices + wave;
  if (lg >= LG) return;
  const size_t row0 = (size_t)lg * N + t0;
  const auto ks = buf_rsrc(K + row0 * D, nb * D * 2);
  const auto rs = buf_rsrc(raw_out + row0 * D, nb * D * 2);
  const int lane_off = (rr * D + cl * 8) * 2;
  u32x4 w[LOADS];
#pragma unroll
  for (int ld = 0; ld < LOADS; ++ld) w[ld] = __builtin_amdgcn_raw_buffer_load_b128(ks, lane_off, ld * kGroupBytes, 0);
  float acc[8] = {kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero};
#pragma unroll
  for (int ld = 0; ld < LOADS; ++ld) {
    const int t = ld * RPL + rr;
    float x[8];
    unpack8(w[ld], x);
    rotate8<D>(x, tab[t], cl, -1);
    buf_store16(pack8(x), rs, lane_off + ld * kGroupBytes);   // whole offset per lane (see buf_store16)
    if (t < nb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  if (rr == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = nb == kBlk ? acc[e] * (1.f / kBlk) : acc[e] / (float)nb;
    store_row_through<D>(index + ((size_t)lg * nB + b) * D, cl, pack8(acc));
  }
}

// Incremental append with de-RoPE stage-out (KVMEM, section "Engineering and
// cost ...": proactive stage-out during chunked prefill, raw K as the
// reconstruction authority; index as in the Mean-K section).  A workgroup owns
// one block the chunk touches and kLgPerWg (layer, KV head) slices of it: it
// builds the block's rotation table once in LDS, removes RoPE from the
// chunk's rows, rounds them to bf16 into the stage, and re-averages the block
// over the staged rows it has so far (earlier rows come from the stage).  The
// sum runs in the same order as meank_build_raw, so the result equals the raw
// build of the stage bit for bit.
constexpr int kLgPerWg = 32;

template <int D>
__global__ __launch_bounds__(256) void meank_append_kernel(const uint16_t* __restrict__ chunk, int64_t n_new,
                                                           int64_t t0, int64_t cap, int64_t nB_cap, int64_t b0,
                                                           int LG, int64_t pos0, double log2_theta,
                                                           uint16_t* __restrict__ stage,
                                                           uint16_t* __restrict__ index) {
  constexpr int LPR = D / 8, RPL = 64 / LPR, LOADS = kBlk / RPL;
  __shared__ float2 tab[kBlk][D / 2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane % LPR, rr = lane / LPR;
  const int64_t b = b0 + blockIdx.x;
  const int64_t tb = b * kBlk;
  const int64_t t1 = t0 + n_new;
  const int nb = (int)min<int64_t>(kBlk, t1 - tb);
  build_rope_table<D>(tab, pos0 + tb, log2_theta);
  __syncthreads();
  const int lg1 = min(LG, (int)(blockIdx.y + 1) * kLgPerWg);
  for (int lg = (int)blockIdx.y * kLgPerWg + wave; lg < lg1; lg += 4) {
    const uint16_t* src = chunk + (size_t)lg * n_new * D + cl * 8;
    uint16_t* st = stage + (size_t)lg * cap * D + cl * 8;
    u32x4 w[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int64_t t = tb + i * RPL + rr;
      w[i] = kNegZeroRows;
      if (t < t0) w[i] = *reinterpret_cast<const u32x4*>(st + (size_t)t * D);
      else if (t < t1) w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)(t - t0) * D));
    }
    float acc[8] = {kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero, kNegZero};
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = i * RPL + rr;
      const int64_t t = tb + r;
      float x[8];
      unpack8(w[i], x);
      rotate8<D>(x, tab[r], cl, -1);        // every lane takes part: rotate8 shuffles
      if (t >= t0 && t < t1) {
        const u32x4 y = pack8(x);
        *reinterpret_cast<u32x4*>(st + (size_t)t * D) = y;
        w[i] = y;
      }
      unpack8(w[i], x);                     // staged (rounded) raw K, -0 past the end
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
    if (rr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = nb == kBlk ? acc[e] * (1.f / kBlk) : acc[e] / (float)nb;
      *reinterpret_cast<u32x4*>(index + ((size_t)lg * nB_cap + b) * D + cl * 8) = pack8(acc);
    }
  }
}

}  // namespace

hipError_t kvs_launch_meank_build(const void* K, int L, int H_kv, int D, int64_t N, int k_is_rope,
                                  int64_t pos0, double theta, void* raw_out, void* index,
                                  hipStream_t st) {
  if (N == 0) return hipSuccess;
  const int64_t nB = (N + kBlk - 1) / kBlk;
  const int LG = L * H_kv;
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  uint16_t* idx = static_cast<uint16_t*>(index);
  if (!k_is_rope) {
    const int64_t total = (int64_t)LG * nB;
    const int64_t wgs = (total + 3) / 4;
    dim3 grid((unsigned)(wgs < (int64_t(1) << 22) ? wgs : (int64_t(1) << 22))), block(256);
    if (D == 128)
      hipLaunchKernelGGL(meank_build_raw<128>, grid, block, 0, st, Kb, N, nB, total, idx);
    else
      hipLaunchKernelGGL(meank_build_raw<64>, grid, block, 0, st, Kb, N, nB, total, idx);
  } else {
    const double l2t = __builtin_log2(theta);
    uint16_t* raw = static_cast<uint16_t*>(raw_out);
    if (raw) {
      dim3 grid((unsigned)(nB * ceil_div(LG, kScatterSlices))), block(kScatterThreads);
      if (D == 128)
        hipLaunchKernelGGL(meank_build_derope_out<128>, grid, block, 0, st, Kb, N, nB, LG, pos0, l2t, raw, idx);
      else
        hipLaunchKernelGGL(meank_build_derope_out<64>, grid, block, 0, st, Kb, N, nB, LG, pos0, l2t, raw, idx);
    } else {
      dim3 grid((unsigned)nB), block(256);
      if (D == 128)
        hipLaunchKernelGGL(meank_build_derope<128>, grid, block, 0, st, Kb, N, nB, LG, pos0, l2t, raw, idx);
      else
        hipLaunchKernelGGL(meank_build_derope<64>, grid, block, 0, st, Kb, N, nB, LG, pos0, l2t, raw, idx);
    }
  }
  return hipGetLastError();
}

hipError_t kvs_launch_meank_append(const void* chunk, int L, int H_kv, int D, int64_t t0, int64_t n_new,
                                   int64_t pos0, double theta, void* stage, int64_t cap, void* index,
                                   hipStream_t st) {
  if (n_new == 0) return hipSuccess;
  const int LG = L * H_kv;
  const int64_t b0 = t0 / kBlk, b1 = (t0 + n_new + kBlk - 1) / kBlk;
  const int64_t nB_cap = (cap + kBlk - 1) / kBlk;
  const double l2t = __builtin_log2(theta);
  const dim3 grid((unsigned)(b1 - b0), ceil_div(LG, kLgPerWg)), block(256);
  const uint16_t* c = static_cast<const uint16_t*>(chunk);
  uint16_t* s = static_cast<uint16_t*>(stage);
  uint16_t* idx = static_cast<uint16_t*>(index);
  if (D == 128)
    hipLaunchKernelGGL(meank_append_kernel<128>, grid, block, 0, st, c, n_new, t0, cap, nB_cap, b0, LG, pos0,
                       l2t, s, idx);
  else
    hipLaunchKernelGGL(meank_append_kernel<64>, grid, block, 0, st, c, n_new, t0, cap, nB_cap, b0, LG, pos0,
                       l2t, s, idx);
  return hipGetLastError();
}
