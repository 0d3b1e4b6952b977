// Rotation table for one 32-token block, shared by the de-RoPE index build,
// the Mean-K append, the re-RoPE scatter and the working-set update.
// Rotate-half pairing (i, i + D/2), omega_i = theta^(-2i/D).  The angle
// p * omega_i is formed in float64 and reduced modulo 2 pi there (at p ~ 1e6 a
// float32 angle would be off by up to ~0.06 rad); the reduced angle, in
// [-pi, pi], goes through float32 sincos, whose few-ulp error is far below the
// bf16 resolution of the rotated keys.
#pragma once

#include "kvs_internal.h"

namespace kvs {

// tab[t][i] = (cos, sin) of (p0 + t) * omega_i for t < 32, i < D/2.  Called by
// all threads of a workgroup whose size is a multiple of D/2, so each thread
// keeps one frequency i.
template <int D>
__device__ __forceinline__ void build_rope_table(float2 (*tab)[D / 2], int64_t p0, double log2_theta) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
  const int i = threadIdx.x % (D / 2);
  const double omega = exp2(-(2.0 * i / D) * log2_theta);
  for (int x = threadIdx.x; x < 32 * (D / 2); x += blockDim.x) {
    const int t = x / (D / 2);
    const double a = (double)(p0 + t) * omega;
    const double r = fma(-rint(a * kInvTwoPi), kTwoPi, a);
    float s, c;
    sincosf((float)r, &s, &c);
    tab[t][i] = make_float2(c, s);
  }
}

// Rotate the 8 coordinates x[] (dims 8*cl .. 8*cl+7 of a D-wide row, with the
// row spread over D/8 lanes) by +angle (dir = +1) or -angle (dir = -1).  All
// lanes of the wave must call this (it shuffles with the partner lane that
// holds dims +- D/2).
template <int D>
__device__ __forceinline__ void rotate8(float* x, const float2* row_tab, int cl, int dir) {
  constexpr int LPR = D / 8;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (LPR == 16)   // partner lane = lane ^ 8: a rotation by 8 within each 16-lane row (DPP)
      p[e] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[e]), 0x128, 0xf, 0xf, false));
    else
      p[e] = __shfl_xor(x[e], LPR / 2, kWave);
  }
  const bool first = cl < LPR / 2;
  // first half: y = x c - dir * xp s ; second half: y = x c + dir * xp s
  const float sg = (first ? -1.f : 1.f) * (float)dir;
  const int i0 = (cl & (LPR / 2 - 1)) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 cs = row_tab[i0 + e];
    x[e] = fmaf(x[e], cs.x, sg * p[e] * cs.y);
  }
}

__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ __forceinline__ u32x4 pack8(const float* x) {
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
               pack_bf16x2(x[6], x[7])};
}

}  // namespace kvs
