// QueryMemory update (IntentKV, Sec. 3.2, Eq. 2):
//   M <- exp(-lambda) M + mean_s q_span[l,h,s,:],  then M[l,h,:] /= ||M[l,h,:]||.
// One wavefront per (layer, query head).  A row of D values is covered by D/8
// lanes with 16-byte (bf16) or 2x16-byte (fp32) loads, so one load instruction
// reads 64/(D/8) rows of the span, and a batch of such loads is in flight at
// once (one wave per head leaves latency, not bandwidth, as the limit).  The
// per-lane partial sums are combined over the row groups with a fixed
// butterfly, the squared norm over the lanes of a row the same way.  The
// previous M row is read first, so its load overlaps the span's.
#include "kvs_internal.h"

using namespace kvs;

namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qmem_kernel(const void* __restrict__ q, int LH, int S,
                                                   float decay, int first_turn,
                                                   float* __restrict__ M) {
  constexpr int LPR = D / 8, RPL = 64 / LPR;
  constexpr int EB = BF16 ? 2 : 4;          // bytes per element
  constexpr int PL = BF16 ? 1 : 2;          // 16-byte loads per lane per row
  constexpr int NB = BF16 ? 16 : 8;         // row groups per batch, all of a batch's loads in flight
  const int lane = threadIdx.x & 63;
  const int lh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lh >= LH) return;
  const int cl = lane % LPR, rr = lane / LPR;
  // the previous M goes out first, so its load overlaps the span's instead of following the sums
  float* m = M + (size_t)lh * D + (size_t)cl * 8;
  float mprev[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mprev[e] = m[e];   // (read on the first turn too, and not used)
  __builtin_amdgcn_sched_barrier(0);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Rows go through a buffer resource over each batch of NB * RPL rows, so the
  // loads of a batch issue together with no branch and rows past S read as
  // zero, which leaves the sums unchanged (they start at +0 and never hold -0);
  // each lane adds its rows in increasing order, as a row-by-row loop would.
  const char* head = static_cast<const char*>(q) + (size_t)lh * S * D * EB;
  for (int s0 = 0; s0 < S; s0 += NB * RPL) {
    const int nrows = min(S - s0, NB * RPL);
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(head + (size_t)s0 * D * EB, nrows * D * EB);
    u32x4 w[NB][PL];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int p = 0; p < PL; ++p)
        w[i][p] = __builtin_amdgcn_raw_buffer_load_b128(rs, ((i * RPL + rr) * D + cl * 8) * EB + 16 * p, 0, 0);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (BF16) {
        const u32x4 v = w[i][0];
        acc[0] += bf16_lo(v.x); acc[1] += bf16_hi(v.x); acc[2] += bf16_lo(v.y); acc[3] += bf16_hi(v.y);
        acc[4] += bf16_lo(v.z); acc[5] += bf16_hi(v.z); acc[6] += bf16_lo(v.w); acc[7] += bf16_hi(v.w);
      } else {
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * p + e] += __uint_as_float(w[i][p][e]);
      }
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  float v[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float enc = acc[e] / (float)S;
    v[e] = first_turn ? enc : fmaf(decay, mprev[e], enc);
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
