// Block relevance R_b (KVMEM, section "Design and trade-offs: step-level
// attention trigger and Mean-K model-native retrieval"): per (layer, query
// head, query token) a softmax over the candidate blocks C of q . kbar / sqrt(D),
// summed over query tokens and averaged over the L*H_q layer-heads.
//
// Per (l, g) this is a dense contraction S = Q_g x index_g^T with Q_g the
// G*Mq query rows of the KV group (contiguous in [L, H_q, Mq, D]) and index_g
// the |C| candidate block means; it runs on bf16 MFMA 32x32x16 with float32
// accumulation.  An exact per-row softmax needs each row's normaliser before
// any column can be summed, and S is far too large to keep, so there are two
// passes over the tiles:
//   1. meank_lse: a wave keeps 32 query rows as the B operand and sweeps the
//      index (A operand).  The tile is S^T, so each lane owns one query row and
//      the online (max, sum 2^(x-max)) stays in-lane.   -> lse2 per row
//   2. meank_colsum: a wave keeps 32 index rows as the B operand and sweeps the
//      query rows (A operand).  Now each lane owns one block column and
//      sum_m 2^(x - lse2[m]) stays in-lane.             -> per-(l,g) partials
//   3. meank_reduce: R_b = sum over (l,g) of the partials, in order, / (L*H_q).
// Operand k-slots: lane half h = lane/32 carries k-slots 8h..8h+7 of every
// k-step; k-step s of half h is dims [64h + 8s, +8) for both operands, so each
// lane reads 128 contiguous bytes of its row.
#include "kvs_internal.h"

using namespace kvs;

namespace {

constexpr int D = 128;
constexpr int KS = D / 16;        // k-steps of the 32x32x16 MFMA
constexpr int kRowsPerWG = 128;   // 4 waves x 32 rows (or columns)

__device__ __forceinline__ void load_operand(const uint16_t* rowp, bool ok, int h, bf16x8* op) {
  const u32x4* p = reinterpret_cast<const u32x4*>(rowp + 64 * h);
#pragma unroll
  for (int s = 0; s < KS; ++s) op[s] = __builtin_bit_cast(bf16x8, ok ? p[s] : u32x4{0u, 0u, 0u, 0u});
}

// C layout of the 32x32 MFMA: lane l holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + (v%4) for v = 0..15.
__device__ __forceinline__ int c_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

__global__ __launch_bounds__(256) void meank_lse(const uint16_t* __restrict__ Q,
                                                 const uint16_t* __restrict__ index, int H_kv, int G,
                                                 int64_t Mq, int64_t nB, int64_t c0, int64_t c1,
                                                 int64_t rows_pad, float scale_log2,
                                                 float* __restrict__ lse2) {
  const int lg = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const int64_t rows = (int64_t)G * Mq;
  const int64_t qrow = (int64_t)blockIdx.x * kRowsPerWG + wave * 32 + n;
  const uint16_t* Qg = Q + (size_t)lg * rows * D;
  const uint16_t* Ig = index + (size_t)lg * nB * D;

  bf16x8 Bq[KS];
  load_operand(Qg + (size_t)(qrow < rows ? qrow : 0) * D, qrow < rows, h, Bq);

  float m = -INFINITY, ssum = 0.f;
  bf16x8 A[KS], An[KS];
  load_operand(Ig + (size_t)min(c0 + n, c1 - 1) * D, c0 + n < c1, h, A);
  for (int64_t cb = c0; cb < c1; cb += 32) {
    const int64_t nb = cb + 32 + n;
    if (cb + 32 < c1) load_operand(Ig + (size_t)min(nb, c1 - 1) * D, nb < c1, h, An);
    f32x16 c = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bq[s], c, 0, 0, 0);
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = cb + c_row(v, h) < c1 ? c[v] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[v]);
    }
    if (tmax != -INFINITY) {
      const float mn = fmaxf(m, tmax);
      float add = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) add += __builtin_amdgcn_exp2f(x[v] - mn);
      ssum = ssum * __builtin_amdgcn_exp2f(m - mn) + add;
      m = mn;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = An[s];
  }
  const float m2 = __shfl_xor(m, 32, kWave);
  const float s2 = __shfl_xor(ssum, 32, kWave);
  lse_merge(m, ssum, m2, s2);
  if (h == 0 && qrow < rows_pad)
    lse2[(size_t)lg * rows_pad + qrow] = (qrow < rows && ssum > 0.f) ? m + log2f(ssum) : INFINITY;
}

__global__ __launch_bounds__(256) void meank_colsum(const uint16_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ index, int G,
                                                    int64_t Mq, int64_t nB, int64_t c0, int64_t c1,
                                                    int64_t rows_pad, float scale_log2,
                                                    const float* __restrict__ lse2,
                                                    float* __restrict__ colpart) {
  const int lg = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const int64_t rows = (int64_t)G * Mq;
  const int64_t col = c0 + (int64_t)blockIdx.x * kRowsPerWG + wave * 32 + n;
  const uint16_t* Qg = Q + (size_t)lg * rows * D;
  const uint16_t* Ig = index + (size_t)lg * nB * D;
  const float* L2 = lse2 + (size_t)lg * rows_pad;

  bf16x8 Bi[KS];
  load_operand(Ig + (size_t)(col < c1 ? col : c0) * D, col < c1, h, Bi);

  float acc = 0.f;
  bf16x8 A[KS], An[KS];
  load_operand(Qg + (size_t)min<int64_t>(n, rows - 1) * D, n < rows, h, A);
  for (int64_t r0 = 0; r0 < rows; r0 += 32) {
    const int64_t nr = r0 + 32 + n;
    if (r0 + 32 < rows) load_operand(Qg + (size_t)min(nr, rows - 1) * D, nr < rows, h, An);
    f32x16 c = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], Bi[s], c, 0, 0, 0);
    // rows r0 + 8u + 4h + 0..3 for u = 0..3 (padding rows hold +inf)
    const float4* lp = reinterpret_cast<const float4*>(L2 + r0 + 4 * h);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 ls = lp[2 * u];
      acc += __builtin_amdgcn_exp2f(fmaf(c[4 * u + 0], scale_log2, -ls.x));
      acc += __builtin_amdgcn_exp2f(fmaf(c[4 * u + 1], scale_log2, -ls.y));
      acc += __builtin_amdgcn_exp2f(fmaf(c[4 * u + 2], scale_log2, -ls.z));
      acc += __builtin_amdgcn_exp2f(fmaf(c[4 * u + 3], scale_log2, -ls.w));
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = An[s];
  }
  acc += __shfl_xor(acc, 32, kWave);
  if (h == 0 && col < c1) colpart[(size_t)lg * nB + col] = acc;
}

__global__ __launch_bounds__(256) void meank_reduce(const float* __restrict__ colpart, int LG,
                                                    int64_t nB, int64_t c0, int64_t c1, float LH, float* __restrict__ R) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nB) return;
  if (b < c0 || b >= c1) { R[b] = 0.f; return; }
  float s = 0.f;
  for (int lg = 0; lg < LG; ++lg) s += colpart[(size_t)lg * nB + b];
  R[b] = s / LH;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t pad32(int64_t x) { return (x + 31) / 32 * 32; }

}  // namespace

size_t kvs_meank_ws_bytes(int L, int H_q, int H_kv, int64_t Mq, int64_t nB) {
  const size_t LG = (size_t)L * H_kv;
  const int64_t rows_pad = pad32((int64_t)(H_q / H_kv) * Mq);
  return align256(LG * (size_t)rows_pad * 4) + align256(LG * (size_t)nB * 4);
}

hipError_t kvs_launch_meank_score(const void* Q, const void* index, int L, int H_q, int H_kv,
                                  int64_t Mq, int64_t nB, int64_t c0, int64_t c1, float* R,
                                  void* ws, hipStream_t st) {
  const int LG = L * H_kv;
  const int G = H_q / H_kv;
  const int64_t rows = (int64_t)G * Mq;
  const int64_t rows_pad = pad32(rows);
  char* w = static_cast<char*>(ws);
  float* lse2 = reinterpret_cast<float*>(w);
  float* colpart = reinterpret_cast<float*>(w + align256((size_t)LG * rows_pad * 4));
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  const uint16_t* Qb = static_cast<const uint16_t*>(Q);
  const uint16_t* Ib = static_cast<const uint16_t*>(index);
  if (c1 > c0 && rows > 0) {
    hipLaunchKernelGGL(meank_lse, dim3(ceil_div(rows_pad, kRowsPerWG), LG), dim3(256), 0, st, Qb, Ib,
                       H_kv, G, Mq, nB, c0, c1, rows_pad, scale_log2, lse2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(meank_colsum, dim3(ceil_div(c1 - c0, kRowsPerWG), LG), dim3(256), 0, st, Qb,
                       Ib, G, Mq, nB, c0, c1, rows_pad, scale_log2, lse2, colpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    c1 = c0;   // no candidates (or no queries): every R_b is 0
  }
  hipLaunchKernelGGL(meank_reduce, dim3(ceil_div(nB, 256)), dim3(256), 0, st, colpart, LG, nB, c0, c1,
                     (float)(L * H_q), R);
  return hipGetLastError();
}
