// QueryMemory update (IntentKV, Sec. 3.2, Eq. 2):
//   M <- exp(-lambda) M + mean_s q_span[l,h,s,:],  then M[l,h,:] /= ||M[l,h,:]||.
// One wavefront per (layer, query head); a lane owns D/64 coordinates.  The
// span is a few MB at most, so the kernel is latency-bound; rows are read
// coalesced (consecutive lanes, consecutive coordinates).
#include "kvs_internal.h"

using namespace kvs;

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qmem_kernel(const void* __restrict__ q, int LH, int S,
                                                   float decay, int first_turn,
                                                   float* __restrict__ M) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x & 63;
  const int lh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (lh >= LH) return;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  const size_t base = (size_t)lh * S * D + (size_t)lane * PER;
  for (int s = 0; s < S; ++s) {
    if constexpr (BF16) {
      const uint16_t* qp = static_cast<const uint16_t*>(q) + base + (size_t)s * D;
#pragma unroll
      for (int p = 0; p < PER; ++p) acc[p] += bf16_to_f32(qp[p]);
    } else {
      const float* qp = static_cast<const float*>(q) + base + (size_t)s * D;
#pragma unroll
      for (int p = 0; p < PER; ++p) acc[p] += qp[p];
    }
  }
  float* m = M + (size_t)lh * D + (size_t)lane * PER;
  float v[PER];
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    float enc = acc[p] / (float)S;
    v[p] = first_turn ? enc : fmaf(decay, m[p], enc);
    ss = fmaf(v[p], v[p], ss);
  }
  ss = wave_sum(ss);
  const float norm = sqrtf(ss);
#pragma unroll
  for (int p = 0; p < PER; ++p) m[p] = ss > 0.f ? v[p] / norm : 0.f;
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
