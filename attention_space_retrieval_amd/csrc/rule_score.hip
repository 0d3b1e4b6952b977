// Rule score (IntentKV, Sec. 3.2, Eqs. 3-4): for each layer l and query head
// h, a softmax over the candidate positions H = [0,N) \ F of
// M[l,h] . K[l,h/G,j] / sqrt(D); rule_j sums the softmaxes over (l, h).
//
// HBM-bound: K is streamed once.  Because every (l, h) softmax has its own
// normaliser, the logits are spilled (fp32, [L*H_q, N]) and summed after the
// normalisers are known:
//   1. rule_logits_*: one workgroup per (chunk of 2048 positions, l, g).  K is
//      streamed in whole rows with non-temporal loads and each 16-row tile is
//      transposed through LDS into the operand of a bf16 MFMA 16x16x32 that
//      computes the G logits of every row; the A operand holds M * log2(e)/sqrt(D) split into a bf16 high part
//      (rows 0..7) and a bf16 low part (rows 8..15), so hi+lo gives the logit
//      to ~2^-16 relative at no extra MFMA cost.  Logits are written in log2
//      units and a per-chunk (max, sum 2^(x-max)) is kept per head.
//   2. rule_lse_merge: per (l, h), merge the chunk partials in order -> lse2.
//   3. rule_colsum: rule_j = sum_{l,h} 2^(x[l,h,j] - lse2[l,h]), fixed order.
// Forced positions carry -inf logits, so they drop out of every softmax and
// their rule value is exactly 0.
#include "kvs_internal.h"

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

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t kvs_rule_ws_bytes(int L, int H_q, int /*H_kv*/, int64_t N) {
  const size_t LH = (size_t)L * H_q;
  const size_t n_chunks = (size_t)ceil_div(N, kChunk);
  return align256(LH * (size_t)N * 4) + align256(LH * n_chunks * 8) + align256(LH * 4);
}

hipError_t kvs_launch_rule(const void* K, int dtype, const int64_t* slots, int64_t pool_size,
                           const float* M, int L, int H_q, int H_kv, int D, int64_t N, int64_t pi,
                           int64_t q_s, int64_t q_e, float* rule, void* ws, hipStream_t st) {
  const int LH = L * H_q;
  const int G = H_q / H_kv;
  const int n_chunks = (int)ceil_div(N, kChunk);
  char* w = static_cast<char*>(ws);
  float* spill = reinterpret_cast<float*>(w);
  w += align256((size_t)LH * (size_t)N * 4);
  float2* partials = reinterpret_cast<float2*>(w);
  w += align256((size_t)LH * n_chunks * 8);
  float* lse2 = reinterpret_cast<float*>(w);
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  const bool paged = slots != nullptr;
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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rule_lse_merge, dim3(ceil_div(LH, 256)), dim3(256), 0, st, partials, LH,
                     n_chunks, lse2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rule_colsum, dim3(ceil_div(N, kColTile)), dim3(256), 0, st, spill, lse2, LH, N,
                     rule);
  return hipGetLastError();
}
