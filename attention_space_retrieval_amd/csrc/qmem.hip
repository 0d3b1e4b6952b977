// QueryMemory update (IntentKV, Sec. 3.2, Eq. 2):
//   M <- exp(-lambda) M + mean_s q_span[l,h,s,:],  then M[l,h,:] /= ||M[l,h,:]||.
// One wavefront per (layer, query head).  A row of D values is covered by D/8
// lanes with 16-byte (bf16) or 2x16-byte (fp32) loads, so one load instruction
// reads 64/(D/8) rows of the span; the per-lane partial sums are combined over
// the row groups with a fixed butterfly, the squared norm over the lanes of a
// row the same way.
#include "kvs_internal.h"

using namespace kvs;

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qmem_kernel(const void* __restrict__ q, int LH, int S,
                                                   float decay, int first_turn,
                                                   float* __restrict__ M) {
  constexpr int LPR = D / 8, RPL = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int lh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (lh >= LH) return;
  const int cl = lane % LPR, rr = lane / LPR;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const size_t base = (size_t)lh * S * D + (size_t)cl * 8;
#pragma unroll 4
  for (int s = rr; s < S; s += RPL) {
    if constexpr (BF16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(q) + base + (size_t)s * D);
      acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x); acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
      acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z); acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(q) + base + (size_t)s * D);
      const float4 a = p[0], b = p[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  float* m = M + (size_t)lh * D + (size_t)cl * 8;
  float v[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float enc = acc[e] / (float)S;
    v[e] = first_turn ? enc : fmaf(decay, m[e], enc);
    ss = fmaf(v[e], v[e], ss);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o, kWave);
  const float norm = sqrtf(ss);
  if (rr == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = ss > 0.f ? v[e] / norm : 0.f;
  }
}

}  // namespace

hipError_t kvs_launch_qmem(const void* q, int dtype, int L, int H_q, int S, int D, float decay,
                           int first_turn, float* M, hipStream_t st) {
  const int LH = L * H_q;
  dim3 grid(ceil_div(LH, 4)), block(256);
  const bool bf = dtype == 1;
  if (D == 128) {
    if (bf) hipLaunchKernelGGL((qmem_kernel<128, true>), grid, block, 0, st, q, LH, S, decay, first_turn, M);
    else hipLaunchKernelGGL((qmem_kernel<128, false>), grid, block, 0, st, q, LH, S, decay, first_turn, M);
  } else {
    if (bf) hipLaunchKernelGGL((qmem_kernel<64, true>), grid, block, 0, st, q, LH, S, decay, first_turn, M);
    else hipLaunchKernelGGL((qmem_kernel<64, false>), grid, block, 0, st, q, LH, S, decay, first_turn, M);
  }
  return hipGetLastError();
}
