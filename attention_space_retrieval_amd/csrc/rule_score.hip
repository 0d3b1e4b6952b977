// Rule score (IntentKV, Sec. 3.2, Eqs. 3-4): for each layer l and query head
// h, a softmax over the candidate positions H = [0,N) \ F of
// M[l,h] . K[l,h/G,j] / sqrt(D); rule_j sums the softmaxes over (l, h).
//
// HBM-bound: K is streamed once.  Every (l, h) softmax has its own
// normaliser, known only once all N positions are scored.  Two forms.
//
// Work-queue fold (bf16 keys, G <= 8): persistent workgroups claim chunks of
// one (l, g) from per-XCD queues.  A workgroup keeps a chunk's logits in LDS,
// publishes the chunk's per-head (max, sum 2^(x-max)), and one chunk later
// folds it: once the group's normalisers are out, it writes one value per
// position, the sum over the G heads of 2^(x - lse2), so only 1/G of the
// per-head values leave the chip.  A chunk whose group is not complete by
// then is spilled instead (per-head logits, as in the spill form) and the
// column sum finishes it; the values are the same bits either way.  Nothing
// ever waits while it holds an unpublished claim: the only blocking wait is
// at the end, after every chunk of every queue has been claimed, and each
// claimed chunk is published by its workgroup before that workgroup waits.
// The wait is bounded as well; past the bound the chunk is spilled.
//
// Spill (float32 keys, or G > 8): the logits are spilled (fp32, [L*H_q, N])
// and summed after the normalisers are known:
//   1. rule_logits_*: one workgroup per (chunk of 2048 positions, l, g).
//   2. rule_lse_merge: per (l, h), merge the chunk partials in order -> lse2.
//   3. rule_colsum: rule_j = sum_{l,h} 2^(x[l,h,j] - lse2[l,h]), fixed order.
//
// In the bf16 kernels K is streamed in whole rows with non-temporal loads and
// each 16-row tile is transposed through LDS into the operand of a bf16 MFMA
// 16x16x32 that computes the G logits of every row; the A operand holds
// M * log2(e)/sqrt(D) split into a bf16 high part (rows 0..7) and a bf16 low
// part (rows 8..15), so hi+lo gives the logit to ~2^-16 relative at no extra
// MFMA cost.  Logits are in log2 units.  Forced positions carry -inf logits,
// so they drop out of every softmax and their rule value is exactly 0.
#include "kvs_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

using namespace kvs;

namespace {

constexpr int kChunk = 2048;   // positions per workgroup in the logit pass
constexpr int kColTile = 64;   // positions per workgroup in the column sum

__device__ __forceinline__ bool is_forced(int64_t j, int64_t pi, int64_t q_s, int64_t q_e) {
  return j < pi || (j >= q_s && j < q_e);
}

__device__ __forceinline__ void online_add(float& m, float& s, float x) {
  const float mn = fmaxf(m, x);
  s = s * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(x - mn);
  m = mn;
}

// online_add that leaves (m, s) unchanged for x = -inf, by selects rather
// than a branch (with m = -inf too, the update would read -inf - -inf).
__device__ __forceinline__ void online_add_live(float& m, float& s, float x) {
  const float mn = fmaxf(m, x);
  const float sn = s * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(x - mn);
  const bool live = x != -INFINITY;
  s = live ? sn : s;
  m = live ? mn : m;
}

// One lane's 8 A-operand values for k-step s: M[head] * log2(e)/sqrt(D) at
// dims d0..d0+7, high bf16 part (hi) or the bf16 rounding of the remainder,
// packed two per register so the operand stays in 4 registers.
__device__ __forceinline__ bf16x8 m_operand(const float* __restrict__ mrow, bool valid, bool hi, int d0,
                                            float scale_log2) {
  u32x4 w = {0u, 0u, 0u, 0u};
  if (valid) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t b[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x = mrow[d0 + e + k] * scale_log2;
        const uint32_t hb = f32_to_bf16_bits(x);
        b[k] = hi ? hb : f32_to_bf16_bits(x - __uint_as_float(hb << 16));
      }
      w[e / 2] = b[0] | (b[1] << 16);
    }
  }
  return __builtin_bit_cast(bf16x8, w);
}

// Paged keys: a token-major pool K_pool[l, slot, g, :] read in place through
// the slot map; a chunk's slots are staged in LDS as int32 (-1 for a slot
// outside the pool, whose position then drops out like a forced one).
template <bool PAGED>
__device__ __forceinline__ void stage_slots(int32_t* sslot, const int64_t* __restrict__ slots, int64_t row0,
                                            int64_t row1, int64_t pool_size) {
  if constexpr (PAGED) {
    for (int64_t j = row0 + threadIdx.x; j < row1; j += 256) {
      const int64_t sl = slots[j];
      sslot[j - row0] = (sl >= 0 && sl < pool_size) ? (int32_t)sl : -1;
    }
    __syncthreads();
  }
}

// NHG = number of 8-head groups (G <= 8*NHG).
template <int D, int NHG, bool PAGED>
__global__ __launch_bounds__(256) void rule_logits_mfma(
    const uint16_t* __restrict__ K, const int64_t* __restrict__ slots, int64_t pool_size,
    const float* __restrict__ M, int H_q, int H_kv, int G,
    int64_t N, int64_t pi, int64_t q_s, int64_t q_e, float scale_log2, float* __restrict__ spill,
    float2* __restrict__ partials, int n_chunks) {
  constexpr int KS = D / 32;            // MFMA k-steps per row
  constexpr int QW = D / 4;             // dims owned by one 16-lane group
  const int chunk = blockIdx.x;
  const int lg = blockIdx.y;
  const int l = lg / H_kv, g = lg - l * H_kv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;

  // A operand: row r of the 16x32 tile is head slot r&7 of group hg, high part
  // for r < 8 and low part for r >= 8; k-slot 8q+e of k-step s is dim q*QW + 8s + e.
  bf16x8 A[NHG][KS];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int hl = hg * 8 + (r & 7);
    const float* mrow = M + ((size_t)l * H_q + (size_t)g * G + hl) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) A[hg][s] = m_operand(mrow, hl < G, r < 8, q * QW + 8 * s, scale_log2);
  }

  float mx[NHG][4], sm[NHG][4];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int v = 0; v < 4; ++v) { mx[hg][v] = -INFINITY; sm[hg][v] = 0.f; }

  const int64_t row0 = (int64_t)chunk * kChunk;
  const int64_t row1 = min(N, row0 + (int64_t)kChunk);
  const uint16_t* Kb = K + (size_t)lg * (size_t)N * D;
  const size_t head0 = (size_t)l * H_q + (size_t)g * G;
  __shared__ int32_t sslot[PAGED ? kChunk : 1];
  stage_slots<PAGED>(sslot, slots, row0, row1, pool_size);
  // K row j of group (l, g), or null when the position has no row in the pool
  auto row_ptr = [&](int64_t j) -> const uint16_t* {
    if constexpr (PAGED) {
      const int32_t sl = sslot[j - row0];
      return sl < 0 ? nullptr : K + (((size_t)l * pool_size + sl) * H_kv + g) * D;
    } else {
      return Kb + (size_t)j * D;
    }
  };

  // K rows are read whole (16 lanes x 16 B = one 256-byte row, 4 rows per
  // instruction) with non-temporal loads: K is touched once, and full-row
  // streaming reads run far closer to the HBM peak than the 64-byte row pieces
  // the MFMA operand layout would need.  Each wave then transposes its 16-row
  // tile through its own padded LDS slot into that layout.
  __shared__ __attribute__((aligned(16))) char stage[4][16 * (D * 2 + 16)];
  constexpr int kRow = D * 2 + 16;
  constexpr int RPI = 64 / (D / 8);                 // rows per load instruction
  constexpr int NLD = 16 / RPI;                     // load instructions per 16-row tile
  char* slot = stage[wave];
  const int lr = lane / (D / 8), lc = lane % (D / 8);
  // Dense keys go through a buffer resource over the chunk's rows, so a row
  // past the chunk reads as zero with no branch: the loads of the next tile
  // then stay in flight while this one is transposed and its logits are
  // written (branchy loads made the compiler wait for every outstanding
  // memory operation, the spill stores included, before each tile).
  const __amdgpu_buffer_rsrc_t krs = buf_rsrc(PAGED ? K : Kb + (size_t)row0 * D, PAGED ? 0 : (int)((row1 - row0) * D * 2));
  auto load_tile = [&](int64_t t0, u32x4* w) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int64_t j = t0 + i * RPI + lr;
      if constexpr (PAGED) {
        const uint16_t* p = j < row1 ? row_ptr(j) : nullptr;
        w[i] = p ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + lc) : u32x4{0u, 0u, 0u, 0u};
      } else {
        w[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(j - row0) * (D * 2) + lc * 16, 0, kBufNt);
      }
    }
  };
  auto to_operand = [&](const u32x4* w, bf16x8* B) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) *reinterpret_cast<u32x4*>(slot + (i * RPI + lr) * kRow + lc * 16) = w[i];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      B[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + r * kRow + (q * QW + 8 * s) * 2));
  };

  u32x4 W[NLD], Wn[NLD];
  bf16x8 B[KS];
  // One 16-row tile: issue the loads of the wave's next tile into nxt, move
  // cur into the operand, and write and fold its logits.
  auto step = [&](int64_t t0, u32x4* cur, u32x4* nxt) {
    if (PAGED ? t0 + 64 < row1 : true) load_tile(t0 + 64, nxt);   // dense: past the chunk the loads return zeros
    to_operand(cur, B);
    const int64_t j = t0 + r;
    const bool vj = j < row1;
    const bool forced = is_forced(j, pi, q_s, q_e) || (PAGED && vj && sslot[j - row0] < 0);
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[hg][s], B[s], c, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // C row 4*(lane>>4)+v: lanes 0..31 hold the high rows, lanes 32..63 the low rows,
        // so lanes 0..15 hold head hg*8+v and lanes 16..31 head hg*8+4+v.
        // lanes 0..31 add the low part held by lane + 32 (v_permlane32_swap hands
        // the upper half-wave's values to the lower half); lanes 32..63 are inactive below
        const uint32_t cu = __float_as_uint(c[v]);
        const float t = c[v] + __uint_as_float(__builtin_amdgcn_permlane32_swap(cu, cu, false, false)[1]);
        const int hl = hg * 8 + 4 * (q & 1) + v;
        const bool act = lane < 32 && vj && hl < G;
        // Branch-free: each head's spill row is a buffer resource (a head past G
        // gets an empty one) and an inactive lane's offset lies out of range, so
        // its store is dropped; a -inf logit leaves the online state as it is.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int hh = hg * 8 + 4 * half + v;
          const __amdgpu_buffer_rsrc_t srs =
              buf_rsrc(spill + (head0 + (hh < G ? hh : 0)) * (size_t)N + row0, hh < G ? (int)((row1 - row0) * 4) : 0);
          const bool mine = act && (q & 1) == half;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(forced ? -INFINITY : t), srs,
                                                mine ? (int)(j - row0) * 4 : 0x7ffffff0, 0, 0);
        }
        online_add_live(mx[hg][v], sm[hg][v], act && !forced ? t : -INFINITY);
      }
    }
  };
  // Tiles alternate between the W and Wn registers (no copies).  The first
  // pair runs before the loop, so every path into the loop head carries the
  // same outstanding memory operations (one tile's loads, then the previous
  // tile's spill stores): the compiler then waits only for the loads a tile
  // needs, not for the stores issued after them.
  int64_t t0 = row0 + wave * 16;
  if (PAGED ? t0 < row1 : true) load_tile(t0, W);
  if (t0 < row1) {
    step(t0, W, Wn);
    if (t0 + 64 < row1) {
      step(t0 + 64, Wn, W);
      for (t0 += 128; t0 < row1; t0 += 128) {
        step(t0, W, Wn);
        if (t0 + 64 >= row1) break;
        step(t0 + 64, Wn, W);
      }
    }
  }

  // Reduce over the 16 lanes that hold the same head, then over the 4 waves.
  __shared__ float2 red[4][NHG * 8];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = __shfl_xor(mx[hg][v], o, kWave);
        const float s2 = __shfl_xor(sm[hg][v], o, kWave);
        lse_merge(mx[hg][v], sm[hg][v], m2, s2);
      }
      if (lane == 0 || lane == 16) red[wave][hg * 8 + 4 * (lane >> 4) + v] = make_float2(mx[hg][v], sm[hg][v]);
    }
  __syncthreads();
  if (threadIdx.x < NHG * 8 && (int)threadIdx.x < G) {
    const int hl = threadIdx.x;
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lse_merge(m, s, red[w][hl].x, red[w][hl].y);
    partials[(head0 + hl) * n_chunks + chunk] = make_float2(m, s);
  }
}

// fp32 keys: plain VALU dot products, one row per thread, same outputs.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void rule_logits_f32(
    const float* __restrict__ K, const int64_t* __restrict__ slots, int64_t pool_size,
    const float* __restrict__ M, int H_q, int H_kv, int G, int64_t N,
    int64_t pi, int64_t q_s, int64_t q_e, float scale_log2, float* __restrict__ spill,
    float2* __restrict__ partials, int n_chunks) {
  constexpr int GMAX = 16;
  __shared__ float Ms[GMAX][D];
  __shared__ float2 red[4][GMAX];
  const int chunk = blockIdx.x;
  const int lg = blockIdx.y;
  const int l = lg / H_kv, g = lg - l * H_kv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t head0 = (size_t)l * H_q + (size_t)g * G;
  for (int i = threadIdx.x; i < G * D; i += 256) Ms[i / D][i % D] = M[head0 * D + i];
  __syncthreads();
  float mx[GMAX], sm[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) { mx[h] = -INFINITY; sm[h] = 0.f; }
  const int64_t row0 = (int64_t)chunk * kChunk;
  const int64_t row1 = min(N, row0 + (int64_t)kChunk);
  const float* Kb = K + (size_t)lg * (size_t)N * D;
  __shared__ int32_t sslot[PAGED ? kChunk : 1];
  stage_slots<PAGED>(sslot, slots, row0, row1, pool_size);
  for (int64_t j = row0 + threadIdx.x; j < row1; j += 256) {
    int32_t sl = 0;
    if constexpr (PAGED) sl = sslot[j - row0];
    const float* krow = PAGED ? K + (((size_t)l * pool_size + (sl < 0 ? 0 : sl)) * H_kv + g) * D
                              : Kb + (size_t)j * D;
    const bool forced = is_forced(j, pi, q_s, q_e) || sl < 0;
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(Ms[h][d], krow[d], dot);
        const float t = dot * scale_log2;
        spill[(head0 + h) * (size_t)N + j] = forced ? -INFINITY : t;
        if (!forced) online_add(mx[h], sm[h], t);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(mx[h], o, kWave);
        const float s2 = __shfl_xor(sm[h], o, kWave);
        lse_merge(mx[h], sm[h], m2, s2);
      }
      if (lane == 0) red[wave][h] = make_float2(mx[h], sm[h]);
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < G) {
    float m = -INFINITY, s = 0.f;
    for (int w = 0; w < 4; ++w) lse_merge(m, s, red[w][threadIdx.x].x, red[w][threadIdx.x].y);
    partials[(head0 + threadIdx.x) * n_chunks + chunk] = make_float2(m, s);
  }
}

__global__ __launch_bounds__(256) void rule_lse_merge(const float2* __restrict__ partials, int LH,
                                                      int n_chunks, float* __restrict__ lse2) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= LH) return;
  float m = -INFINITY, s = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    const float2 p = partials[(size_t)i * n_chunks + c];
    lse_merge(m, s, p.x, p.y);
  }
  lse2[i] = s > 0.f ? m + log2f(s) : INFINITY;
}

__global__ __launch_bounds__(256) void rule_colsum(const float* __restrict__ spill,
                                                   const float* __restrict__ lse2, int LH, int64_t N,
                                                   float* __restrict__ rule) {
  __shared__ float part[4][kColTile];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * kColTile + lane;
  float acc = 0.f;
  if (j < N) {
    const float* col = spill + j;
#pragma unroll 8
    for (int lh = wave; lh < LH; lh += 4)
      acc += __builtin_amdgcn_exp2f(col[(size_t)lh * N] - lse2[lh]);
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && j < N) rule[j] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

// ---------------------------------------------------------------------------
// Work-queue fold (bf16 keys, G <= 8).

constexpr int kQueues = 2;                       // claim counters, each shared by half the workgroups
constexpr int kLine = 64;                        // words between counters (one 256-byte line each)
constexpr int kFoldWaves = 4;                    // waves per workgroup
constexpr int kFoldThreads = 64 * kFoldWaves;
constexpr uint32_t kLseUnset = 0x7fbadbadu;      // a NaN payload no arithmetic here produces
constexpr uint32_t kNanBits = 0x7fc00000u;       // the canonical quiet NaN
// A chunk partial is the bit pair (max, sum); a sum is never negative, so
// (0, -1) marks a slot not yet published.
constexpr uint64_t kPartUnset = (uint64_t)0xbf800000u << 32;
// A chunk is settled this many chunks after it was scored, so that the
// other chunks of its group, claimed about when it was, are published by
// then.  Each chunk held costs LDS, and a longer lag with shorter chunks ran
// slower (the fixed costs of a chunk dominate below 512 positions).
constexpr int kFoldLag = 1;

__device__ __forceinline__ uint64_t part_bits(float m, float s) {
  return (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(s) << 32);
}

// Normalisers of the heads h0, h0 + hs, ... (at most HM of them, all < G)
// of one group from their chunk partials, by one wave: lane i merges chunks
// i, i+64, i+128, ... in that order, then an xor butterfly merges the lanes;
// lse[h] takes lane 0's value.  The loads of a batch of 64*KB chunks of all
// the heads go out together.  False if a partial is still unpublished (the
// results are then meaningless).  part: [G][n_chunks] words of the group.
template <int HM, int KB = 4>
__device__ bool group_lse(const uint64_t* part, int n_chunks, int h0, int hs, int G, int lane, float* lse) {
  float m[HM], s[HM];
#pragma unroll
  for (int j = 0; j < HM; ++j) { m[j] = -INFINITY; s[j] = 0.f; }
  bool miss = false;
  for (int c0 = 0; c0 < n_chunks; c0 += 64 * KB) {
    uint64_t w[HM][KB];
#pragma unroll
    for (int j = 0; j < HM; ++j) {
      const int h = h0 + j * hs;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int c = c0 + 64 * k + lane;
        w[j][k] = (h < G && c < n_chunks)
                      ? __hip_atomic_load(part + (size_t)h * n_chunks + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : part_bits(-INFINITY, 0.f);
      }
    }
#pragma unroll
    for (int j = 0; j < HM; ++j)
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float pm = __uint_as_float((uint32_t)w[j][k]), ps = __uint_as_float((uint32_t)(w[j][k] >> 32));
        miss |= ps < 0.f;
        lse_merge(m[j], s[j], pm, ps < 0.f ? 0.f : ps);
      }
  }
#pragma unroll
  for (int j = 0; j < HM; ++j) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m[j], o, kWave);
      const float s2 = __shfl_xor(s[j], o, kWave);
      lse_merge(m[j], s[j], m2, s2);
    }
    float v = s[j] > 0.f ? m[j] + log2f(s[j]) : INFINITY;
    v = v != v ? __uint_as_float(kNanBits) : v;
    const int h = h0 + j * hs;
    if (h < G) lse[h] = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
  }
  return __ballot(miss) == 0;
}

struct FoldArgs {
  const uint16_t* K;
  const int64_t* slots;
  int64_t pool_size;
  const float* M;
  int H_q, H_kv, G, LHkv;
  int64_t N, pi, q_s, q_e;
  float scale_log2;
  int n_chunks;
  int64_t spin;            // bounded waits, in polls; < 0: no chunk is folded (every one is spilled)
  float* spill;            // [L*H_q][N]
  uint64_t* partials;      // [L*H_q][n_chunks]
  uint32_t* lse;           // [L*H_kv][kLine]: the G normaliser bits of a group at the start of its
                           // line, kLseUnset until a workgroup has merged them
  float* fold;             // [L*H_kv][N]
  uint32_t* spilled;       // [n_chunks][L*H_kv]: 1 = the chunk went to the spill
  uint32_t* count;         // [L*H_kv][kLine]: chunks published per group (word 0 of each line)
  uint32_t* queue;         // [kQueues][kLine]: claims handed out per queue (word 0 of each line)
};

// Items of queue qi: the groups qi, qi + kQueues, ... chunk by chunk.
__device__ __forceinline__ uint32_t queue_items(const FoldArgs& a, int qi) {
  return qi < a.LHkv ? (uint32_t)((a.LHkv - qi + kQueues - 1) / kQueues) * (uint32_t)a.n_chunks : 0u;
}

// CP positions per chunk (a multiple of 64: each of the 4 waves takes every
// fourth 16-row tile).  held: [kFoldLag + 1][G][CP + 4] floats of dynamic
// LDS; the +4 puts the heads 4 apart that the two half-waves write on
// different banks.
//
// A workgroup holds the kFoldLag chunks it scored last.  One pass of the
// loop, for the claimed chunk: its tiles (during the second-last one the
// next ticket is taken and the normalisers and publish count of the oldest
// held chunk's group are fetched), its partials out, the next chunk's first
// loads, then the oldest held chunk settled: folded with the published
// normalisers, or with normalisers this workgroup merges itself when every
// chunk of the group has counted itself published (and publishes them for
// the others), or else spilled.  Nothing waits inside the loop (a complete
// group's partials are only polled for until they land).
//
// The one wait is at a workgroup's end, once its claim comes back empty:
// every chunk of every queue has been claimed then, and each is published by
// its workgroup before that one can reach this wait.  It is bounded besides;
// past the bound the chunk is spilled.
//
// WPS: workgroups per CU that the LDS footprint allows (2 or 3); the register
// budget is cut for the waves per SIMD that makes.  With fewer waves per SIMD,
// each keeps more 16-row tiles of K in flight (4 instead of 2).
template <int D, bool PAGED, int CP, int WPS>
__global__ __launch_bounds__(kFoldThreads, WPS * kFoldWaves / 4) void rule_fold_queue(FoldArgs a) {
  constexpr int LAG = kFoldLag;
  constexpr int KS = D / 32;            // MFMA k-steps per row
  constexpr int QW = D / 4;             // dims owned by one 16-lane group
  constexpr int HS = CP + 4;            // held-logit row stride
  constexpr int NT = CP / (16 * kFoldWaves);   // 16-row tiles per wave per chunk
  static_assert(CP % (16 * kFoldWaves) == 0, "a chunk is whole rounds of the waves' tiles");
  constexpr int HPW = 8 / kFoldWaves;   // heads per wave when the waves merge a group's normalisers
  constexpr int kRow = D * 2 + 16;
  constexpr int RPI = 64 / (D / 8);     // rows per load instruction
  constexpr int NLD = 16 / RPI;         // load instructions per 16-row tile
  static_assert(NT >= 2, "the fetches ride on the second-last tile");
  extern __shared__ float held[];
  __shared__ __attribute__((aligned(16))) char stage[kFoldWaves][16 * kRow];
  __shared__ float2 red[kFoldWaves][8];
  __shared__ float s_lse[8];
  __shared__ int s_lg, s_c, s_pub, s_cmp;
  __shared__ int s_miss[2][kFoldWaves];
  __shared__ int32_t sslot[PAGED ? CP : 1];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int G = a.G;
  const int nc = a.n_chunks;
  const int64_t N = a.N;
  char* slot = stage[wave];
  const int lr = lane / (D / 8), lc = lane % (D / 8);

  // Claims, by thread 0: a ticket of queue pq is taken early and resolved
  // later; a queue found empty moves the workgroup on to the next one.
  const int home = blockIdx.x % kQueues;
  int pq = home, qoff = 0;
  uint32_t ticket = 0;
  auto take = [&]() {
    ticket = __hip_atomic_fetch_add(a.queue + (size_t)pq * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto resolve = [&]() {
    for (;;) {
      if (ticket < queue_items(a, pq)) {
        s_lg = pq + kQueues * (int)(ticket / (uint32_t)nc);
        s_c = (int)(ticket % (uint32_t)nc);
        return;
      }
      if (++qoff == kQueues) {
        s_lg = -1;
        return;
      }
      pq = (home + qoff) % kQueues;
      take();
    }
  };

  // Per-chunk operands: M of the group as the A operand, the chunk's rows.
  bf16x8 A[KS];
  int l = 0, g = 0;
  int64_t row0 = 0, row1 = 0;
  __amdgpu_buffer_rsrc_t krs = buf_rsrc(a.K, 0);
  auto setup = [&](int lg_, int c_) {
    l = lg_ / a.H_kv;
    g = lg_ - l * a.H_kv;
    const int hl = r & 7;
    const float* mrow = a.M + ((size_t)lg_ * G + hl) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = m_operand(mrow, hl < G, r < 8, q * QW + 8 * s, a.scale_log2);
    row0 = (int64_t)c_ * CP;
    row1 = min(N, row0 + (int64_t)CP);
    if constexpr (!PAGED) krs = buf_rsrc(a.K + ((size_t)lg_ * (size_t)N + (size_t)row0) * D, (int)((row1 - row0) * D * 2));
  };
  // Paged: a chunk's slots, read into registers early and staged in LDS later
  // (as int32, -1 for a slot outside the pool).
  constexpr int SPT = (CP + kFoldThreads - 1) / kFoldThreads;
  int64_t slot_reg[PAGED ? SPT : 1];
  auto read_slots = [&](int c_) {
    if constexpr (PAGED) {
      const int64_t r0 = (int64_t)c_ * CP, r1 = min(N, r0 + (int64_t)CP);
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const int64_t j = r0 + threadIdx.x + k * kFoldThreads;
        slot_reg[k] = j < r1 ? a.slots[j] : -1;
      }
    }
  };
  auto stage_slots = [&]() {
    if constexpr (PAGED) {
#pragma unroll
      for (int k = 0; k < SPT; ++k) {
        const int i = threadIdx.x + k * kFoldThreads;
        if (i < CP) sslot[i] = (slot_reg[k] >= 0 && slot_reg[k] < a.pool_size) ? (int32_t)slot_reg[k] : -1;
      }
    }
  };
  auto load_tile = [&](int64_t t0, u32x4* w) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int64_t j = t0 + i * RPI + lr;
      if constexpr (PAGED) {
        const int32_t sl = j < row1 ? sslot[j - row0] : -1;
        w[i] = sl >= 0 ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4*>(a.K + (((size_t)l * a.pool_size + sl) * a.H_kv + g) * D) + lc)
                       : u32x4{0u, 0u, 0u, 0u};
      } else {
        // past the chunk the loads return zeros
        w[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(j - row0) * (D * 2) + lc * 16, 0, kBufNt);
      }
    }
  };

  // Settle the held chunk c of group lg from hb: fold it, or spill it.
  // s_pub: its normalisers were already out (in s_lse); s_cmp: every chunk of
  // the group had counted itself published.  last: the workgroup's final
  // chunk, which may wait.  Every wave takes part; the decision is uniform.
  auto settle = [&](int lg, int c, const float* hb, bool last) {
    bool ok = s_pub != 0;
    if (!ok && (s_cmp || last)) {
      const uint64_t* part = a.partials + (size_t)lg * G * nc;
      for (int64_t it = 0;; ++it) {
        float lse[8];
        const bool mine = group_lse<HPW>(part, nc, wave, kFoldWaves, G, lane, lse);
        if (lane == 0) {
#pragma unroll
          for (int j = 0; j < HPW; ++j)
            if (wave + j * kFoldWaves < G) s_lse[wave + j * kFoldWaves] = lse[wave + j * kFoldWaves];
          s_miss[it & 1][wave] = !mine;
        }
        __syncthreads();
        int miss = 0;
#pragma unroll
        for (int w = 0; w < kFoldWaves; ++w) miss |= s_miss[it & 1][w];
        ok = !miss;
        if (ok) {
          // publish for the other workgroups of the group (the same bits whoever merges)
          if (lane == 0) {
#pragma unroll
            for (int j = 0; j < HPW; ++j) {
              const int h = wave + j * kFoldWaves;
              if (h < G)
                __hip_atomic_store(a.lse + (size_t)lg * kLine + h, __float_as_uint(lse[h]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
          }
          break;
        }
        if (it >= a.spin) break;
        __builtin_amdgcn_s_sleep(2);
      }
    }
    ok = ok && a.spin >= 0;             // a negative limit folds nothing (the normalisers still go out)
    const int head0 = lg * G;
    const int64_t r0 = (int64_t)c * CP;
    const int nrow = (int)(min(N, r0 + (int64_t)CP) - r0);
    if (ok) {
      // written through to memory (device scope): inside the saturated K stream
      // this costs less than write-back stores (rule-14b: 1.643 vs 1.677 ms)
      uint32_t* out = reinterpret_cast<uint32_t*>(a.fold + (size_t)lg * N + r0);
      for (int p = threadIdx.x; p < nrow; p += kFoldThreads) {
        float e = 0.f;
        for (int h = 0; h < G; ++h) e += __builtin_amdgcn_exp2f(hb[h * HS + p] - s_lse[h]);
        __hip_atomic_store(out + p, __float_as_uint(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      for (int h = 0; h < G; ++h) {
        float* out = a.spill + ((size_t)head0 + h) * N + r0;
        for (int p = threadIdx.x; p < nrow; p += kFoldThreads) out[p] = hb[h * HS + p];
      }
      if (threadIdx.x == 0) a.spilled[(size_t)c * a.LHkv + lg] = 1u;
    }
  };

  if (threadIdx.x == 0) {
    take();
    resolve();
  }
  __syncthreads();
  int lg = __builtin_amdgcn_readfirstlane(s_lg), c = __builtin_amdgcn_readfirstlane(s_c);
  if (lg < 0) return;
  constexpr int RING = WPS * kFoldWaves / 4 <= 2 ? 4 : 2;   // more tiles in flight when fewer waves share a SIMD
  constexpr int PF = RING < NT ? RING : NT;
  u32x4 W[PF][NLD];
  bf16x8 B[KS];
  auto first_loads = [&]() {
#pragma unroll
    for (int i = 0; i + 1 < PF; ++i) load_tile(row0 + wave * 16 + 16 * kFoldWaves * i, W[i]);
  };
  read_slots(c);
  stage_slots();
  setup(lg, c);
  if constexpr (PAGED) __syncthreads();
  first_loads();
  // Held chunks, most recent first, with their buffers; buffer bcur takes the claimed chunk.
  int h_lg[LAG], h_c[LAG], h_b[LAG];
#pragma unroll
  for (int k = 0; k < LAG; ++k) { h_lg[k] = -1; h_c[k] = 0; h_b[k] = k + 1; }
  int bcur = 0;
  for (;;) {
    float* hb = held + bcur * G * HS;
    const int old_lg = h_lg[LAG - 1];
    float mx[4], sm[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) { mx[v] = -INFINITY; sm[v] = 0.f; }
    uint32_t lsev = 0;                  // wave 0: lanes < G normaliser bits, lane 63 the publish count,
                                        // of the held chunk's group
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int64_t t0 = row0 + wave * 16 + 16 * kFoldWaves * i;
      if (i + PF - 1 < NT) load_tile(t0 + 16 * kFoldWaves * (PF - 1), W[(i + PF - 1) % PF]);
      if (i == NT - 2) {
        if (threadIdx.x == 0) take();
        if (wave == 0 && old_lg >= 0 && (lane < G || lane == 63))
          lsev = __hip_atomic_load(lane < G ? a.lse + (size_t)old_lg * kLine + lane : a.count + (size_t)old_lg * kLine,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int k = 0; k < NLD; ++k) *reinterpret_cast<u32x4*>(slot + (k * RPI + lr) * kRow + lc * 16) = W[i % PF][k];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        B[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slot + r * kRow + (q * QW + 8 * s) * 2));
      const int64_t j = t0 + r;
      const bool vj = j < row1;
      const bool forced = is_forced(j, a.pi, a.q_s, a.q_e) || (PAGED && vj && sslot[j - row0] < 0);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s], B[s], acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // C row 4*(lane>>4)+v: lanes 0..15 hold head v, lanes 16..31 head 4+v
        // (high parts); v_permlane32_swap brings the low parts from lanes 32..63.
        const uint32_t cu = __float_as_uint(acc[v]);
        const float t = acc[v] + __uint_as_float(__builtin_amdgcn_permlane32_swap(cu, cu, false, false)[1]);
        const int hl = 4 * (q & 1) + v;
        const bool act = lane < 32 && vj && hl < G;
        if (act) hb[hl * HS + (int)(j - row0)] = forced ? -INFINITY : t;
        online_add_live(mx[v], sm[v], act && !forced ? t : -INFINITY);
      }
    }
    if (threadIdx.x == 0) resolve();    // the ticket went out two tiles ago
    // Chunk partials: reduce over the 16 lanes of a head, then over the 4 waves.
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = __shfl_xor(mx[v], o, kWave);
        const float s2 = __shfl_xor(sm[v], o, kWave);
        lse_merge(mx[v], sm[v], m2, s2);
      }
      if (lane == 0 || lane == 16) red[wave][4 * (lane >> 4) + v] = make_float2(mx[v], sm[v]);
    }
    __syncthreads();
    const int nlg = __builtin_amdgcn_readfirstlane(s_lg), ncc = __builtin_amdgcn_readfirstlane(s_c);
    if (nlg >= 0) read_slots(ncc);
    if (wave == 0) {
      if (lane < G) {
        float m = -INFINITY, s = 0.f;
#pragma unroll
        for (int w = 0; w < kFoldWaves; ++w) lse_merge(m, s, red[w][lane].x, red[w][lane].y);
        __hip_atomic_store(a.partials + ((size_t)lg * G + lane) * nc + c, part_bits(m, s), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane == 0) __hip_atomic_fetch_add(a.count + (size_t)lg * kLine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old_lg >= 0) {
        bool pub = __ballot(lane < G && lsev == kLseUnset) == 0;
        bool cmp = __builtin_amdgcn_readlane(lsev, 63) >= (uint32_t)nc;
        if (!pub && !cmp) {             // look once more: the group may have completed since
          lsev = (lane < G || lane == 63)
                     ? __hip_atomic_load(lane < G ? a.lse + (size_t)old_lg * kLine + lane : a.count + (size_t)old_lg * kLine,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : 0u;
          pub = __ballot(lane < G && lsev == kLseUnset) == 0;
          cmp = __builtin_amdgcn_readlane(lsev, 63) >= (uint32_t)nc;
        }
        if (lane < 8) s_lse[lane] = __uint_as_float(lsev);
        if (lane == 0) {
          s_pub = pub;
          s_cmp = cmp;
        }
      }
    }
    if (nlg >= 0) stage_slots();        // this chunk's tiles are done with the slots
    __syncthreads();
    if (nlg >= 0) {
      setup(nlg, ncc);
      first_loads();
    }
    if (old_lg >= 0) settle(old_lg, h_c[LAG - 1], held + h_b[LAG - 1] * G * HS, false);
    const int freed = h_b[LAG - 1];
#pragma unroll
    for (int k = LAG - 1; k > 0; --k) { h_lg[k] = h_lg[k - 1]; h_c[k] = h_c[k - 1]; h_b[k] = h_b[k - 1]; }
    h_lg[0] = lg;
    h_c[0] = c;
    h_b[0] = bcur;
    bcur = freed;
    if (nlg < 0) break;
    lg = nlg;
    c = ncc;
    __syncthreads();                    // the held chunk is settled before the next tiles overwrite its buffer
  }

  // No claim is pending: every chunk is claimed.  Settle the held chunks, oldest first.
#pragma unroll
  for (int k = LAG - 1; k >= 0; --k) {
    if (h_lg[k] < 0) continue;
    __syncthreads();
    if (threadIdx.x == 0) s_pub = s_cmp = 0;
    __syncthreads();
    settle(h_lg[k], h_c[k], held + h_b[k] * G * HS, true);
  }
}

// Workspace state of the fold, cleared before every call (a kernel, not a
// memset, so a captured graph replays it).
__global__ __launch_bounds__(256) void rule_fold_reset(uint64_t* __restrict__ partials, int64_t n_part,
                                                       uint32_t* __restrict__ lse, uint32_t* __restrict__ spilled,
                                                       int64_t n_spilled, uint32_t* __restrict__ count, int LHkv,
                                                       uint32_t* __restrict__ queue) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n_part) partials[i] = kPartUnset;
  if (i < (int64_t)LHkv * kLine) {
    lse[i] = kLseUnset;
    count[i] = 0u;
  }
  if (i < n_spilled) spilled[i] = 0u;
  if (i < kQueues * kLine) queue[i] = 0u;
}

// rule_j = sum over the L*H_kv groups, in a fixed order, of the folded value,
// or, for a chunk that went to the spill, of the same sum of the G heads'
// terms computed here from the spilled logits.  VEC * 64 positions per
// workgroup, all in one chunk (the chunk length is a multiple of that), VEC
// consecutive positions per lane (VEC = 4 when N is a multiple of 4, so each
// load instruction reads 1 KB of a row).  Sixteen waves split the groups of a
// workgroup's positions, so each wave's chain of dependent load rounds is a
// sixteenth of the rows long: wave w takes the groups w, w+16, ..., their
// spill flags arriving 64 at a time in one load and the folded values 8 rows
// at a time, before any of them is needed; the wave sums are then added in
// wave order.  (Four waves, each walking a quarter of the rows, took 39 us
// instead of 27 at L*H_kv = 384, N = 92160.)  The rare spill branch merges a
// group's normalisers one head at a time, which keeps the kernel at 92
// registers, so sixteen waves fit without spilling.
constexpr int kColWaves = 16;                   // waves per column-sum workgroup
template <int VEC>
__global__ __launch_bounds__(64 * kColWaves) void rule_fold_colsum(const float* __restrict__ fold,
                                                        const float* __restrict__ spill,
                                                        const uint64_t* __restrict__ partials,
                                                        const uint32_t* __restrict__ lse,
                                                        const uint32_t* __restrict__ spilled, int LHkv, int G,
                                                        int n_chunks, int CP, int64_t N, float* __restrict__ rule) {
  constexpr int RB = 8;                 // rows per batch of loads
  using VT = std::conditional_t<VEC == 4, u32x4, uint32_t>;
  __shared__ float part[kColWaves][64 * VEC];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t j0 = (int64_t)blockIdx.x * (64 * VEC);
  const int64_t j = j0 + (int64_t)lane * VEC;   // the lane's first position; past N a row reads as zero
  const int c = (int)(j0 / CP);
  const uint32_t* flags = spilled + (size_t)c * LHkv;
  const int rows = (LHkv - wave + kColWaves - 1) / kColWaves;   // this wave's groups: wave + kColWaves*k, k < rows
  // one row of N floats as a buffer resource; offsets past it read zero
  auto load_row = [&](const float* row) -> VT {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(row, (int)(N * 4));
    if constexpr (VEC == 4) return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(j * 4), 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(j * 4), 0, 0);
  };
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < rows; k0 += 64) {
    const int kk = k0 + lane;
    const uint32_t fl = kk < rows ? flags[wave + kColWaves * kk] : 0u;   // lane i: the flag of the wave's row k0 + i
    const int nb = min(64, rows - k0);
    for (int b0 = 0; b0 < nb; b0 += RB) {
      VT fv[RB];
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        const int lg = wave + kColWaves * (k0 + min(b0 + t, nb - 1));
        fv[t] = load_row(fold + (size_t)lg * N);
      }
#pragma unroll
      for (int t = 0; t < RB; ++t) {
        if (b0 + t >= nb) break;
        const int lg = wave + kColWaves * (k0 + b0 + t);
        float v[VEC];
        if constexpr (VEC == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(fv[t][e]);
        } else {
          v[0] = __uint_as_float(fv[t]);
        }
        if (__builtin_amdgcn_readlane(fl, b0 + t)) {
          const int head0 = lg * G;
          float L[8];
          bool have = true;
#pragma unroll
          for (int hl = 0; hl < 8; ++hl) {
            const uint32_t bits = hl < G ? __builtin_amdgcn_readfirstlane(lse[(size_t)lg * kLine + hl]) : 0u;
            L[hl] = __uint_as_float(bits);
            have &= hl >= G || bits != kLseUnset;
          }
          // Normalisers never published: no chunk of this group was folded, so
          // computing them here is consistent (and gives the same bits anyway).
          // one head at a time (the merge order, and so the bits, do not depend on the batching)
          if (!have) {
#pragma unroll
            for (int hl = 0; hl < 8; ++hl)
              if (hl < G) group_lse<1, 1>(partials + (size_t)head0 * n_chunks, n_chunks, hl, 1, G, lane, L);
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = 0.f;
          for (int h = 0; h < G; ++h) {
            const VT x = load_row(spill + ((size_t)head0 + h) * N);
            if constexpr (VEC == 4) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += __builtin_amdgcn_exp2f(__uint_as_float(x[e]) - L[h]);
            } else {
              v[0] += __builtin_amdgcn_exp2f(__uint_as_float(x) - L[h]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += v[e];
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[wave][lane * VEC + e] = acc[e];
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * VEC; i += 64 * kColWaves) {
    const int64_t jj = j0 + i;
    float r = part[0][i];
#pragma unroll
    for (int w = 1; w < kColWaves; ++w) r += part[w][i];
    if (jj < N) rule[jj] = r;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Fold chunk length.  Dense keys: the largest whose kFoldLag + 1 held
// buffers of G*(CP+4) floats fit 42 KB (two or three workgroups per CU:
// longer chunks beat more workgroups there).  Paged keys: the largest that
// still leaves three workgroups per CU beside the chunk's slot array (the
// gathered rows want the occupancy more).  The transpose stage is counted at
// its D = 128 size.
inline int fold_chunk(int G, bool paged) {
  for (int cp : {1024, 768, 512, 256}) {
    const size_t held = (size_t)(kFoldLag + 1) * G * (cp + 4) * 4;
    if (!paged ? held <= 43008 : held + 4 * 16 * 272 + (size_t)cp * 4 + 512 <= 160 * 1024 / 3) return cp;
  }
  return 256;
}
// Chunks per group the workspace is sized for: the shorter of the two chunk lengths.
inline int64_t fold_chunks_max(int G, int64_t N) {
  return (int64_t)ceil_div(N, std::min(fold_chunk(G, false), fold_chunk(G, true)));
}

// Compute units of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workspace regions.  The spill and its partials serve both forms; the rest
// only the fold.
struct RuleWs {
  float* spill;
  void* partials;         // spill form: float2 [LH][chunks of 2048]; fold: uint64 [LH][chunks of CP]
  float* lse2;            // spill form: [LH] float; fold: [LH] normaliser bits
  float* fold;
  uint32_t* spilled;
  uint32_t* count;
  uint32_t* queue;
  size_t bytes;
};

RuleWs rule_ws(void* base, int L, int H_q, int H_kv, int64_t N) {
  const size_t LH = (size_t)L * H_q, LHkv = (size_t)L * H_kv;
  const int G = H_q / H_kv;
  const size_t nc_spill = (size_t)ceil_div(N, kChunk);
  const size_t nc_fold = G <= 8 ? (size_t)fold_chunks_max(G, N) : 0;
  const bool fold = G <= 8;
  char* w = static_cast<char*>(base);
  size_t off = 0;
  RuleWs r;
  auto take = [&](size_t bytes) { void* p = w ? w + off : nullptr; off += align256(bytes); return p; };
  r.spill = static_cast<float*>(take(LH * (size_t)N * 4));
  r.partials = take(LH * (nc_spill > nc_fold ? nc_spill : nc_fold) * 8);
  r.lse2 = static_cast<float*>(take(LH * 4 > LHkv * kLine * 4 ? LH * 4 : LHkv * kLine * 4));
  r.fold = static_cast<float*>(take(fold ? LHkv * (size_t)N * 4 : 0));
  r.spilled = static_cast<uint32_t*>(take(fold ? LHkv * nc_fold * 4 : 0));
  r.count = static_cast<uint32_t*>(take(fold ? LHkv * kLine * 4 : 0));
  r.queue = static_cast<uint32_t*>(take(fold ? kQueues * kLine * 4 : 0));
  r.bytes = off;
  return r;
}

std::atomic<int64_t> g_fold_spin{1 << 14};

}  // namespace

int64_t kvs_rule_fold_spin(int64_t polls) { return g_fold_spin.exchange(polls); }

size_t kvs_rule_ws_bytes(int L, int H_q, int H_kv, int64_t N) {
  return rule_ws(nullptr, L, H_q, H_kv, N).bytes;
}

hipError_t kvs_launch_rule(const void* K, int dtype, const int64_t* slots, int64_t pool_size,
                           const float* M, int L, int H_q, int H_kv, int D, int64_t N, int64_t pi,
                           int64_t q_s, int64_t q_e, float* rule, void* ws, hipStream_t st) {
  const int LH = L * H_q;
  const int LHkv = L * H_kv;
  const int G = H_q / H_kv;
  const RuleWs w = rule_ws(ws, L, H_q, H_kv, N);
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  const bool paged = slots != nullptr;
  hipError_t e;

  const int CP = G <= 8 ? fold_chunk(G, paged) : 0;
  const int64_t nc_fold = CP ? (int64_t)ceil_div(N, CP) : 0;
  if (dtype == 1 && G <= 8 && (int64_t)LHkv * nc_fold < ((int64_t)1 << 30)) {
    const int64_t n_part = (int64_t)LH * nc_fold;
    uint64_t* partials = static_cast<uint64_t*>(w.partials);
    uint32_t* lse = reinterpret_cast<uint32_t*>(w.lse2);
    const int64_t n_reset = std::max<int64_t>(std::max<int64_t>(n_part, (int64_t)LHkv * kLine), kQueues * kLine);
    hipLaunchKernelGGL(rule_fold_reset, dim3(ceil_div(n_reset, 256)), dim3(256), 0, st, partials, n_part, lse,
                       w.spilled, (int64_t)LHkv * nc_fold, w.count, LHkv, w.queue);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    FoldArgs a;
    a.K = static_cast<const uint16_t*>(K);
    a.slots = slots;
    a.pool_size = pool_size;
    a.M = M;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = G;
    a.LHkv = LHkv;
    a.N = N;
    a.pi = pi;
    a.q_s = q_s;
    a.q_e = q_e;
    a.scale_log2 = scale_log2;
    a.n_chunks = (int)nc_fold;
    a.spin = g_fold_spin.load();
    a.spill = w.spill;
    a.partials = partials;
    a.lse = lse;
    a.fold = w.fold;
    a.spilled = w.spilled;
    a.count = w.count;
    a.queue = w.queue;
    const int64_t items = (int64_t)LHkv * nc_fold;
    const size_t lds = (size_t)(kFoldLag + 1) * G * (CP + 4) * 4;
    // the kernel's own LDS: the transpose stage, the slots of a paged chunk, a few words
    const size_t lds_static = (size_t)kFoldWaves * 16 * (2 * D + 16) + (paged ? (size_t)CP * 4 : 0) + 512;
    const int wps = (int)((160 * 1024) / (lds + lds_static));
    // one resident wave of persistent workgroups (a multiple of kQueues)
    const int64_t resident = (int64_t)device_cus() * std::min(std::max(wps, 1), 3) / kQueues * kQueues;
    const unsigned grid = (unsigned)std::max<int64_t>(kQueues, std::min(resident, (items + kQueues - 1) / kQueues * kQueues));
#define FOLD_LAUNCH(DD, PG, CC)                                                                          \
  do {                                                                                                  \
    if (wps >= 3) hipLaunchKernelGGL((rule_fold_queue<DD, PG, CC, 3>), dim3(grid), dim3(kFoldThreads), lds, st, a); \
    else hipLaunchKernelGGL((rule_fold_queue<DD, PG, CC, 2>), dim3(grid), dim3(kFoldThreads), lds, st, a);          \
  } while (0)
#define FOLD_LAUNCH_C(DD, PG)                                                             \
  switch (CP) {                                                                           \
    case 1024: FOLD_LAUNCH(DD, PG, 1024); break;                                          \
    case 768: FOLD_LAUNCH(DD, PG, 768); break;                                            \
    case 512: FOLD_LAUNCH(DD, PG, 512); break;                                            \
    default: FOLD_LAUNCH(DD, PG, 256); break;                                             \
  }
    if (D == 128) { if (paged) { FOLD_LAUNCH_C(128, true) } else { FOLD_LAUNCH_C(128, false) } }
    else { if (paged) { FOLD_LAUNCH_C(64, true) } else { FOLD_LAUNCH_C(64, false) } }
#undef FOLD_LAUNCH_C
#undef FOLD_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (N % 4 == 0)
      hipLaunchKernelGGL(rule_fold_colsum<4>, dim3(ceil_div(N, 4 * 64)), dim3(64 * kColWaves), 0, st, w.fold, w.spill, partials,
                         lse, w.spilled, LHkv, G, (int)nc_fold, CP, N, rule);
    else
      hipLaunchKernelGGL(rule_fold_colsum<1>, dim3(ceil_div(N, 64)), dim3(64 * kColWaves), 0, st, w.fold, w.spill, partials,
                         lse, w.spilled, LHkv, G, (int)nc_fold, CP, N, rule);
    return hipGetLastError();
  }

  const int n_chunks = (int)ceil_div(N, kChunk);
  float* spill = w.spill;
  float2* partials = static_cast<float2*>(w.partials);
  float* lse2 = w.lse2;
  dim3 grid(n_chunks, L * H_kv), block(256);
  if (dtype == 1) {
    const uint16_t* Kb = static_cast<const uint16_t*>(K);
#define RULE_LAUNCH(DD, NH, PG)                                                                     \
  hipLaunchKernelGGL((rule_logits_mfma<DD, NH, PG>), grid, block, 0, st, Kb, slots, pool_size, M, H_q, \
                     H_kv, G, N, pi, q_s, q_e, scale_log2, spill, partials, n_chunks)
#define RULE_LAUNCH_D(DD) \
  if (paged) { if (G <= 8) RULE_LAUNCH(DD, 1, true); else RULE_LAUNCH(DD, 2, true); } \
  else { if (G <= 8) RULE_LAUNCH(DD, 1, false); else RULE_LAUNCH(DD, 2, false); }
    if (D == 128) { RULE_LAUNCH_D(128) } else { RULE_LAUNCH_D(64) }
#undef RULE_LAUNCH_D
#undef RULE_LAUNCH
  } else {
    const float* Kf = static_cast<const float*>(K);
#define RULE_F32(DD, PG)                                                                            \
  hipLaunchKernelGGL((rule_logits_f32<DD, PG>), grid, block, 0, st, Kf, slots, pool_size, M, H_q, H_kv, \
                     G, N, pi, q_s, q_e, scale_log2, spill, partials, n_chunks)
    if (D == 128) { if (paged) RULE_F32(128, true); else RULE_F32(128, false); }
    else { if (paged) RULE_F32(64, true); else RULE_F32(64, false); }
#undef RULE_F32
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rule_lse_merge, dim3(ceil_div(LH, 256)), dim3(256), 0, st, partials, LH,
                     n_chunks, lse2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rule_colsum, dim3(ceil_div(N, kColTile)), dim3(256), 0, st, spill, lse2, LH, N,
                     rule);
  return hipGetLastError();
}
