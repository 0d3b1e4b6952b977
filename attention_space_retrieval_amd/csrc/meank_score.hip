// Block relevance R_b (KVMEM, section "Design and trade-offs: step-level
// attention trigger and Mean-K model-native retrieval"): per (layer, query
// head, query token) a softmax over the candidate blocks C of q . kbar / sqrt(D),
// summed over query tokens and averaged over the L*H_q layer-heads.
//
// Per (l, g) this is a dense contraction S = Q_g x index_g^T with Q_g the
// G*Mq query rows of the KV group (contiguous in [L, H_q, Mq, D]) and index_g
// the |C| candidate block means, on bf16 MFMA 32x32x16 with float32
// accumulation.  An exact per-row softmax needs each row's normaliser before
// any column can be summed and S is far too large to keep, so the tiles are
// computed twice:
//   pass 1 (lse):    persistent operand = 64 query rows per wave, streamed =
//                    32-block index tiles.  C = index_tile x Q^T, so a lane
//                    owns one query row and its online (max, sum 2^(x-max))
//                    is reduced in-lane.                -> lse2[row]
//   pass 2 (colsum): persistent operand = 64 index rows per wave, streamed =
//                    32-row query tiles (+ their lse2).  C = Q_tile x index^T,
//                    so a lane owns one block column and
//                    sum_m 2^(x - lse2[m]) is in-lane.  -> per-(l,g) partials
//   reduce:          R_b = sum of the (l,g) partials in fixed order / (L*H_q).
// Both passes share one engine: a 256-thread workgroup keeps 256 persistent
// rows in registers, streams 8 KB tiles global -> LDS (double buffered, rows
// padded to 272 bytes so the 16-byte MFMA operand reads are bank-conflict free
// and use immediate offsets) and software-pipelines each wave: each MFMA of
// tile t+1 is followed by a slice of tile t's exp2 epilogue, so the matrix and
// vector units overlap.  The same engine serves the window score (the SnapKV
// window of query rows over the cache's keys; see the end of this file).  R_b
// at D = 128 runs meank_pass_dma, the same pipeline with the streamed tiles
// brought into LDS by load-to-LDS DMA (below).
// Workgroups are mapped XCD-aware: the tiles of one (l, g) land on the same
// XCD and share its L2 copy of the streamed operand.
// Operand k-slots: lane half h = lane/32 carries k-slots 8h..8h+7 of every
// k-step; k-step s of half h is dims [h*D/2 + 8s, +8) for both operands, so a
// lane reads one contiguous half row.  The engine is built for D = 128 and
// D = 64 (D/16 k-steps of the 32x32x16 MFMA per tile).
#include <type_traits>

#include "kvs_internal.h"

using namespace kvs;

namespace {

constexpr int kTile = 32;           // streamed rows per tile
constexpr int kPerWave = 64;        // persistent rows per wave (two 32-row operands)
constexpr int kPerWG = 4 * kPerWave;
constexpr float kRebase = 0x1p60f;        // pass 1 rebases its reference past this tile sum

// Per head dimension: k-steps of the 32x32x16 MFMA, row bytes, and the padded
// LDS row (row stride = 16 mod 128 bytes, so the 16-byte operand reads of 16
// consecutive rows hit 16 distinct bank groups: conflict-free).
template <int D>
struct Dims {
  static_assert(D == 64 || D == 128, "head dimension");
  static constexpr int KS = D / 16;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte pieces per row
  static constexpr int kLdsRow = kRowBytes + 16;
  static constexpr int kTileBytes = kTile * kRowBytes;
  static constexpr int EPS = 16 / KS;                   // logits of each C tile per MFMA in the epilogue
};

// C layout of the 32x32 MFMA: lane l holds column l%32 and rows
// 8*(v/4) + 4*(l/32) + (v%4) for v = 0..15.
__device__ __forceinline__ int c_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// NT = threads per workgroup: a tile of 32 rows is kTileBytes / 16 pieces of 16 bytes.
template <int D, int NT>
struct Stage {
  u32x4 w[Dims<D>::kTileBytes / 16 / NT];
  float4 lse;
};

// Global -> registers for streamed tile k: rows [32k, 32k+32) of a buffer
// resource over the streamed rows (and, with lse, one over their lse2).  Rows
// past the resource read as zero, so the loads need no branch: every tile,
// the partial last one and those past the end alike, issues the same loads,
// which lets the compiler keep a later tile's loads in flight while it waits
// for an earlier one.
template <bool WITH_LSE, int D, int NT>
__device__ __forceinline__ void stage_load(Stage<D, NT>& st, __amdgpu_buffer_rsrc_t rows, int k,
                                           __amdgpu_buffer_rsrc_t lse) {
  const int t = threadIdx.x;
  const int base = k * Dims<D>::kTileBytes;
#pragma unroll
  for (int i = 0; i < Dims<D>::kTileBytes / 16 / NT; ++i)
    st.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rows, base + (t + NT * i) * 16, 0, 0);
  if (WITH_LSE) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lse, t < 8 ? (k * kTile + 4 * t) * 4 : 0x7ffffff0, 0, 0);
    st.lse = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
  }
}

template <bool WITH_LSE, int D, int NT>
__device__ __forceinline__ void stage_store(const Stage<D, NT>& st, char* buf, float* lbuf) {
  using Dm = Dims<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Dm::kTileBytes / 16 / NT; ++i) {
    const int idx = t + NT * i, row = idx / Dm::kChunks, chunk = idx % Dm::kChunks;
    *reinterpret_cast<u32x4*>(buf + row * Dm::kLdsRow + chunk * 16) = st.w[i];
  }
  if (WITH_LSE && t < 8) *reinterpret_cast<float4*>(lbuf + 4 * t) = st.lse;
}

template <int D>
__device__ __forceinline__ void read_streamed(const char* buf, int lane, bf16x8* A) {
  using Dm = Dims<D>;
  const char* p = buf + (lane & 31) * Dm::kLdsRow + (lane >> 5) * (Dm::kRowBytes / 2);
#pragma unroll
  for (int s = 0; s < Dm::KS; ++s) A[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + 16 * s));
}

__device__ __forceinline__ void read_lse16(const float* lbuf, int h, float* l16) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 v4 = *reinterpret_cast<const float4*>(lbuf + 8 * u + 4 * h);
    l16[4 * u] = v4.x; l16[4 * u + 1] = v4.y; l16[4 * u + 2] = v4.z; l16[4 * u + 3] = v4.w;
  }
}

template <int D>
__device__ __forceinline__ void mma2(const bf16x8* A, const bf16x8* B0, const bf16x8* B1, f32x16& c0,
                                     f32x16& c1) {
  c0 = f32x16{};
  c1 = f32x16{};
#pragma unroll
  for (int s = 0; s < Dims<D>::KS; ++s) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B0[s], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B1[s], c1, 0, 0, 0);
  }
}

__device__ __forceinline__ float tile_max(const f32x16& c) {
  float t = fmaxf(fmaxf(c[0], c[1]), c[2]);
#pragma unroll
  for (int v = 3; v < 15; v += 2) t = fmaxf(fmaxf(t, c[v]), c[v + 1]);
  return fmaxf(t, c[15]);
}

// Pins a value to this point of the instruction stream (an empty asm that
// claims to read and rewrite it), so IR passes cannot sink the epilogue slice
// below the MFMAs it is meant to overlap.
#define KVS_PIN2(a, b) asm volatile("" : "+v"(a), "+v"(b))

// One software-pipelined step: the 2*D/16 MFMAs of the next tile (cn = A x B)
// are issued one at a time, each followed by a slice of the current tile's
// epilogue (EPS = 16/(D/16) logits of each C tile: 2 at D = 128, 4 at D = 64),
// with scheduling barriers in between so the matrix unit works while the
// wave's vector ALU runs the exp2 epilogue.  ref0/ref1 are the per-lane
// exponent references (pass 1: the running reference of the lane's query row;
// pass 2: unused, the row lse2 in l16).
template <bool PASS1, int D>
__device__ __forceinline__ void step_mma_epi(const bf16x8* A, const bf16x8* B0, const bf16x8* B1,
                                             f32x16& cn0, f32x16& cn1, const f32x16& cc0,
                                             const f32x16& cc1, float scale, const float* l16,
                                             float ref0, float ref1, float& sum0, float& sum1) {
  constexpr int KS = Dims<D>::KS, EPS = Dims<D>::EPS;
  cn0 = f32x16{};
  cn1 = f32x16{};
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    cn0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B0[s], cn0, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EPS; e += 2) {
      const int v = EPS * s + e;
      a0 += __builtin_amdgcn_exp2f(fmaf(cc0[v], scale, -(PASS1 ? ref0 : l16[v])));
      a1 += __builtin_amdgcn_exp2f(fmaf(cc0[v + 1], scale, -(PASS1 ? ref0 : l16[v + 1])));
    }
    KVS_PIN2(a0, a1);
    __builtin_amdgcn_sched_barrier(0);
    cn1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[s], B1[s], cn1, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EPS; e += 2) {
      const int v = EPS * s + e;
      b0 += __builtin_amdgcn_exp2f(fmaf(cc1[v], scale, -(PASS1 ? ref1 : l16[v])));
      b1 += __builtin_amdgcn_exp2f(fmaf(cc1[v + 1], scale, -(PASS1 ? ref1 : l16[v + 1])));
    }
    KVS_PIN2(b0, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  sum0 = a0 + a1;
  sum1 = b0 + b1;
}

// Pass-1 accumulation of one C tile's sum `a` taken against reference m.  The
// reference only moves when a tile could overflow: then the tile is redone
// against its exact max (rare; terms below 2^-126 of the reference are
// negligible against the terms that set it).  MASK tiles (the last one, or
// one that meets the excluded span [h0, h1)) are always redone with the
// positions past c1 or inside the span taken out.
template <bool MASK>
__device__ __forceinline__ void lse_fold(const f32x16& c, float scale, float& m, float& s, float a,
                                         int64_t b0, int h, int64_t c1, int64_t h0, int64_t h1) {
  if (MASK || !(a <= kRebase)) {
    float x[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t pos = b0 + c_row(v, h);
      x[v] = (MASK && (pos >= c1 || (pos >= h0 && pos < h1))) ? -INFINITY : c[v];
    }
    float t = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
    for (int v = 3; v < 15; v += 2) t = fmaxf(fmaxf(t, x[v]), x[v + 1]);
    t = fmaxf(t, x[15]);
    const float mn = fmaxf(fmaxf(m, t * scale), -3.0e38f);
    a = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) a += __builtin_amdgcn_exp2f(fmaf(x[v], scale, -mn));
    s = fmaf(s, __builtin_amdgcn_exp2f(m - mn), a);
    m = mn;
  } else {
    s += a;
  }
}

// blockIdx.x -> (lg, tile) so that one lg's tiles share an XCD (dispatch is
// round-robin over the 8 XCDs).  Falls back to the plain order when LG % 8 != 0.
__device__ __forceinline__ void xcd_map(int T, int LG, int& lg, int& tile) {
  const int w = blockIdx.x;
  if ((LG & 7) == 0) {
    const int x = w & 7, j = w >> 3;
    lg = x + 8 * (j / T);
    tile = j % T;
  } else {
    lg = w / T;
    tile = w % T;
  }
}

// Columns (streamed in pass 1, persistent in pass 2) are the candidates
// [c0, c1).  With SPAN (the window score) they also exclude [h0, h1), and
// pass 1 may split the candidate range over n_split workgroups (gridDim.y);
// each then writes a (max, sum) partial per row to part1 and meank_lse_merge
// combines them.  R_b instantiates SPAN = false, which compiles both out.
template <bool PASS1, bool SPAN, int NW, int D>
__global__ __launch_bounds__(64 * NW, 2) void meank_pass(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ index, int LG,
                                                     int64_t rows, int64_t rows_pad, int64_t nB,
                                                     int64_t c0, int64_t c1, int64_t h0, int64_t h1,
                                                     int T, float scale, int n_split,
                                                     float* __restrict__ lse2,
                                                     float2* __restrict__ part1,
                                                     float* __restrict__ colpart) {
  using Dm = Dims<D>;
  constexpr int KS = Dm::KS, kRowBytes = Dm::kRowBytes, kLdsRow = Dm::kLdsRow;
  constexpr int NT = 64 * NW, PER_WG = NW * kPerWave;   // threads and persistent rows per workgroup
  // one LDS area: first the workgroup's persistent rows, then the two streamed tiles
  __shared__ __attribute__((aligned(16))) char smem[PER_WG * kLdsRow];
  __shared__ __attribute__((aligned(16))) float lses[2][kTile];
  char(*tiles)[kTile * kLdsRow] = reinterpret_cast<char(*)[kTile * kLdsRow]>(smem);
  int lg, tile;
  xcd_map(T, LG, lg, tile);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const uint16_t* Qg = Q + (size_t)lg * rows * D;
  const uint16_t* Ig = index + (size_t)lg * nB * D;
  const float* Lg = lse2 + (size_t)lg * rows_pad;

  const int64_t p0 = (int64_t)tile * PER_WG + wave * kPerWave;   // the wave's first persistent row
  // streamed operand: pass 1 = index tiles over this split of [c0, c1), pass 2 = query tiles over [0, rows)
  const uint16_t* sbase = PASS1 ? Ig : Qg;
  int64_t s_begin = PASS1 ? c0 : 0, s_end = PASS1 ? c1 : rows;
  if (!SPAN) { h0 = 0; h1 = 0; n_split = 1; }
  if (PASS1 && SPAN && n_split > 1) {
    const int64_t span = ((c1 - c0 + n_split - 1) / n_split + kTile - 1) / kTile * kTile;
    s_begin = c0 + span * blockIdx.y;
    s_end = min(c1, s_begin + span);
    if (s_begin >= s_end) {             // nothing left for this split: an empty partial
      if (h == 0) {
        const int64_t r0 = p0 + n, r1 = p0 + 32 + n;
        if (r0 < rows_pad) part1[((size_t)lg * rows_pad + r0) * n_split + blockIdx.y] = make_float2(-INFINITY, 0.f);
        if (r1 < rows_pad) part1[((size_t)lg * rows_pad + r1) * n_split + blockIdx.y] = make_float2(-INFINITY, 0.f);
      }
      return;
    }
  }
  const int nt = (int)((s_end - s_begin + kTile - 1) / kTile);

  // Tiles reach LDS two at a time (double buffer); global loads run ahead of
  // them in a ring of PF register stages, so a tile's load is issued PF - 1
  // iterations before its LDS store.  R_b's pass 1 streams index blocks from
  // HBM and takes the deeper ring (about 1% faster); pass 2 streams L2-resident
  // query tiles, and the window score's pass 1 gains nothing from it.
  constexpr int PF = (PASS1 && !SPAN) ? 4 : 2;
  // streamed rows [s_begin, s_end) and, in pass 2, their lse2 (tile k = rows 32k..)
  const __amdgpu_buffer_rsrc_t srows = buf_rsrc(sbase + (size_t)s_begin * D, (int)((s_end - s_begin) * kRowBytes));
  const __amdgpu_buffer_rsrc_t slse = buf_rsrc(Lg, PASS1 ? 0 : (int)(rows_pad * 4));
  // The first two streamed tiles' loads go out before the persistent rows':
  // a workgroup that streams few tiles (the window score's pass 2 streams
  // four or five) would otherwise wait for them one after the other once
  // its persistent rows are in.
  Stage<D, NT> st[PF];
  stage_load<!PASS1>(st[0], srows, 0, slse);
  stage_load<!PASS1>(st[1], srows, 1, slse);
  // persistent operand: pass 1 = query rows, pass 2 = index rows (block columns).
  // The workgroup's 256 rows are read whole and coalesced (16 loads of 16 bytes
  // per thread at D = 128; rows past the end read as zero), staged in LDS, and each wave
  // takes its 64 rows in the operand layout from there.  Loaded straight in
  // that layout, every load instruction would touch 64 rows 16 bytes at a
  // time, which starves the passes that stream few tiles per workgroup.
  bf16x8 B0[KS], B1[KS];
  {
    const int64_t pbase = (PASS1 ? 0 : c0) + (int64_t)tile * PER_WG;
    const int64_t plim = PASS1 ? rows : c1;
    const int pcount = (int)(plim <= pbase ? 0 : (plim - pbase > PER_WG ? PER_WG : plim - pbase));
    const uint16_t* pg = (PASS1 ? Qg : Ig) + (pcount > 0 ? (size_t)pbase * D : 0);
    const __amdgpu_buffer_rsrc_t prs = buf_rsrc(pg, pcount * kRowBytes);
    constexpr int kLoads = PER_WG * kRowBytes / 16 / NT;
    u32x4 v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(prs, (threadIdx.x + NT * i) * 16, 0, 0);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = threadIdx.x + NT * i;
      *reinterpret_cast<u32x4*>(smem + (idx / Dm::kChunks) * kLdsRow + (idx % Dm::kChunks) * 16) = v[i];
    }
    __syncthreads();
    const char* r0 = smem + (wave * kPerWave + n) * kLdsRow + h * (kRowBytes / 2);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      B0[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(r0 + 16 * k));
      B1[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(r0 + 32 * kLdsRow + 16 * k));
    }
    __syncthreads();
  }
  stage_store<!PASS1>(st[0], tiles[0], lses[0]);
  stage_store<!PASS1>(st[1], tiles[1], lses[1]);
#pragma unroll
  for (int k = 2; k <= PF; ++k) stage_load<!PASS1>(st[k % PF], srows, k, slse);
  __syncthreads();

  // A wave whose persistent rows all lie past the end (the window score's
  // G*W query rows fill half a workgroup) skips the tiles' MFMAs and
  // epilogue; it still stages tiles and meets every barrier, and writes nothing.
  const bool live = p0 < (PASS1 ? rows : c1 - c0);   // wave-uniform
  bf16x8 A[KS];
  f32x16 cA0 = {}, cA1 = {}, cB0 = {}, cB1 = {};     // ping-pong accumulators (tile t and t+1)
  float lA[16], lB[16];               // pass 2: lse2 of the rows of tile t and t+1
  read_streamed<D>(tiles[0], lane, A);
  if (!PASS1) read_lse16(lses[0], h, lA);
  if (live) mma2<D>(A, B0, B1, cA0, cA1);
  __syncthreads();

  // pass 1: running reference and sum per persistent row; pass 2: column sums
  float m0, m1, s0 = 0.f, s1 = 0.f;
  if (PASS1) {
    // the first tile may also be the partial last one, or meet the excluded span: mask those columns
    f32x16 x0 = cA0, x1 = cA1;
    if (SPAN || nt == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t pos = s_begin + c_row(v, h);
        if (pos >= s_end || (SPAN && pos >= h0 && pos < h1)) { x0[v] = -INFINITY; x1[v] = -INFINITY; }
      }
    }
    m0 = fmaxf(tile_max(x0) * scale, -3.0e38f);
    m1 = fmaxf(tile_max(x1) * scale, -3.0e38f);
    m0 = fmaxf(m0, __shfl_xor(m0, 32, kWave));        // both halves share the row's reference
    m1 = fmaxf(m1, __shfl_xor(m1, 32, kWave));
  }

  // Process tile t (accumulators cc, lse lc) while issuing tile t+1 into cn;
  // load tile t+1+PF into stage sl = st[(t+1) % PF] and move tile t+2, loaded
  // PF-1 iterations earlier, from stage ss = st[(t+2) % PF] into LDS.
  auto body = [&](int t, f32x16& cc0, f32x16& cc1, float* lc, f32x16& cn0, f32x16& cn1, float* ln,
                  Stage<D, NT>& sl, Stage<D, NT>& ss) __attribute__((always_inline)) {
    const bool pre = t + 2 < nt;
    stage_load<!PASS1>(sl, srows, t + 1 + PF, slse);   // past the end: reads nothing, returns zeros
    read_streamed<D>(tiles[(t + 1) & 1], lane, A);
    if (!PASS1) read_lse16(lses[(t + 1) & 1], h, ln);
    float a0 = 0.f, a1 = 0.f;
    if (live) step_mma_epi<PASS1, D>(A, B0, B1, cn0, cn1, cc0, cc1, scale, lc, m0, m1, a0, a1);
    if (PASS1) {
      const int64_t tb = s_begin + (int64_t)t * kTile;
      if (SPAN && tb < h1 && tb + kTile > h0) {    // tile meets the excluded span (wave-uniform)
        lse_fold<true>(cc0, scale, m0, s0, a0, tb, h, s_end, h0, h1);
        lse_fold<true>(cc1, scale, m1, s1, a1, tb, h, s_end, h0, h1);
      } else if (__builtin_expect(__ballot(!(a0 <= kRebase) || !(a1 <= kRebase)) != 0, 0)) {
        // rebase only when some lane's tile sum could overflow (wave-uniform, rare)
        lse_fold<false>(cc0, scale, m0, s0, a0, 0, h, c1, h0, h1);
        lse_fold<false>(cc1, scale, m1, s1, a1, 0, h, c1, h0, h1);
      } else {
        s0 += a0;
        s1 += a1;
      }
    } else {
      s0 += a0;
      s1 += a1;
    }
    if (pre) stage_store<!PASS1>(ss, tiles[t & 1], lses[t & 1]);
    __syncthreads();
  };

  // Even t computes into the B accumulators, odd t into A; the loop runs PF
  // tiles per trip so every stage index is a constant, then the up to PF - 1
  // tiles left start at a multiple of PF as well.
  // kc: t % PF as a type, so every stage index is a constant; always inlined,
  // since a call would move the accumulators and stages to scratch memory
  auto body_k = [&](int t, auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr ((k & 1) != 0) body(t, cB0, cB1, lB, cA0, cA1, lA, st[(k + 1) % PF], st[(k + 2) % PF]);
    else body(t, cA0, cA1, lA, cB0, cB1, lB, st[(k + 1) % PF], st[(k + 2) % PF]);
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;
  int t = 0;
  for (; t + PF < nt; t += PF) {
    body_k(t, K0{});
    body_k(t + 1, K1{});
    if constexpr (PF == 4) {
      body_k(t + 2, K2{});
      body_k(t + 3, K3{});
    }
  }
  if (t + 1 < nt) {
    body_k(t, K0{});
    if constexpr (PF == 4) {
      if (t + 2 < nt) {
        body_k(t + 1, K1{});
        if (t + 3 < nt) body_k(t + 2, K2{});
      }
    }
  }
  // the last tile, nt - 1, was computed by body nt - 2 (B if that is even), or by the prologue
  const bool last_b = nt >= 2 && (nt & 1) == 0;
  f32x16* last0 = last_b ? &cB0 : &cA0;
  f32x16* last1 = last_b ? &cB1 : &cA1;
  float* llast = last_b ? lB : lA;
  // last tile (the only one that can be partial)
  if (PASS1) {
    const int64_t b0 = s_begin + (int64_t)(nt - 1) * kTile;
    lse_fold<true>(*last0, scale, m0, s0, 0.f, b0, h, s_end, h0, h1);
    lse_fold<true>(*last1, scale, m1, s1, 0.f, b0, h, s_end, h0, h1);
  } else {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      a0 += __builtin_amdgcn_exp2f(fmaf((*last0)[v], scale, -llast[v]));
      a1 += __builtin_amdgcn_exp2f(fmaf((*last1)[v], scale, -llast[v]));
    }
    s0 += a0;
    s1 += a1;
  }

  if (PASS1) {
    float mm = __shfl_xor(m0, 32, kWave), ss = __shfl_xor(s0, 32, kWave);
    lse_merge(m0, s0, mm, ss);
    mm = __shfl_xor(m1, 32, kWave);
    ss = __shfl_xor(s1, 32, kWave);
    lse_merge(m1, s1, mm, ss);
    if (h == 0) {
      const int64_t r0 = p0 + n, r1 = p0 + 32 + n;
      if (SPAN && n_split > 1) {
        if (r0 < rows_pad) part1[((size_t)lg * rows_pad + r0) * n_split + blockIdx.y] = make_float2(m0, s0);
        if (r1 < rows_pad) part1[((size_t)lg * rows_pad + r1) * n_split + blockIdx.y] = make_float2(m1, s1);
      } else {
        if (r0 < rows_pad) lse2[(size_t)lg * rows_pad + r0] = (r0 < rows && s0 > 0.f) ? m0 + log2f(s0) : INFINITY;
        if (r1 < rows_pad) lse2[(size_t)lg * rows_pad + r1] = (r1 < rows && s1 > 0.f) ? m1 + log2f(s1) : INFINITY;
      }
    }
  } else {
    s0 += __shfl_xor(s0, 32, kWave);
    s1 += __shfl_xor(s1, 32, kWave);
    if (h == 0) {
      const int64_t b0 = c0 + p0 + n, b1 = c0 + p0 + 32 + n;
      if (b0 < c1) colpart[(size_t)lg * nB + b0] = s0;
      if (b1 < c1) colpart[(size_t)lg * nB + b1] = s1;
    }
  }
}

// R_b's passes with the streamed tiles fed to LDS by load-to-LDS DMA
// (`buffer_load_dwordx4 ... lds`, gfx950) instead of through a ring of
// register stages and LDS stores.  Each lane's 16 bytes land at the
// instruction's LDS base + 16 * lane, from any global offset the lane names,
// so a tile is laid out unpadded (32 rows of 256 bytes) with chunk c of row r
// at chunk position c ^ (r & 15): the operand reads of 16 consecutive rows
// then still hit 16 distinct bank groups.  kDmaBufs tiles are in flight;
// tile k is issued kDmaBufs - 1 tiles ahead of its use, each wave waits for
// its own part of the next tile with an explicit vmcnt (nothing else in the
// loop touches vector memory), and a bare s_barrier (no fence, which would
// wait for every outstanding DMA) publishes it.  A row past the end of the
// streamed rows reads as zero.  The persistent operand is loaded straight in
// operand layout: it is read once per workgroup, against hundreds of
// streamed tiles.  D = 128 only.  Same-process A/B against meank_pass, same
// bits: meank-256k 5.00 -> 4.86 ms, meank-1m 39.4 -> 38.2 ms (a ring of six
// tiles measured level with four); with the lane's operand offsets computed
// once (each buffer's base in the read's immediate offset) and the tile's
// offset in the DMA's scalar offset, a further 1-1.4%.
constexpr int kDmaBufs = 4;

// One load-to-LDS DMA of 16 bytes a lane: lane l's bytes go to lds + 16 * l, from the lane's
// offset voff plus the wave-uniform offset soff.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

template <bool PASS1>
__global__ __launch_bounds__(256, 2) void meank_pass_dma(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ index, int LG,
                                                         int64_t rows, int64_t rows_pad, int64_t nB,
                                                         int64_t c0, int64_t c1, int T, float scale,
                                                         float* __restrict__ lse2, float* __restrict__ colpart) {
  constexpr int D = 128;
  using Dm = Dims<D>;
  constexpr int KS = Dm::KS, kRowBytes = Dm::kRowBytes, kChunks = Dm::kChunks;
  constexpr int NT = 256, PER_WG = 4 * kPerWave;
  // DMA instructions a wave issues per tile: its two 1 KB quarters of the tile, and in pass 2
  // its 32-byte quarter of the tile's lse2 (two lanes)
  constexpr int kPerTile = PASS1 ? 2 : 3;
  __shared__ __attribute__((aligned(16))) char tb0[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) char tb1[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) char tb2[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) char tb3[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) float lb0[kTile];
  __shared__ __attribute__((aligned(16))) float lb1[kTile];
  __shared__ __attribute__((aligned(16))) float lb2[kTile];
  __shared__ __attribute__((aligned(16))) float lb3[kTile];
  int lg, tile;
  xcd_map(T, LG, lg, tile);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const uint16_t* Qg = Q + (size_t)lg * rows * D;
  const uint16_t* Ig = index + (size_t)lg * nB * D;
  const float* Lg = lse2 + (size_t)lg * rows_pad;
  const int64_t p0 = (int64_t)tile * PER_WG + wave * kPerWave;   // the wave's first persistent row

  const uint16_t* sbase = PASS1 ? Ig : Qg;
  const int64_t s_begin = PASS1 ? c0 : 0, s_end = PASS1 ? c1 : rows;
  const int nt = (int)((s_end - s_begin + kTile - 1) / kTile);
  const __amdgpu_buffer_rsrc_t srows = buf_rsrc(sbase + (size_t)s_begin * D, (int)((s_end - s_begin) * kRowBytes));
  const __amdgpu_buffer_rsrc_t slse = buf_rsrc(Lg, PASS1 ? 0 : (int)(rows_pad * 4));
  // this lane's global byte offsets within a tile for its two DMA quarters (rows 4q .. 4q+3 of
  // quarter q = 2 * wave + i, chunk position lane & 15 holding chunk (lane & 15) ^ (row & 15))
  int goff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * wave + i) + (lane >> 4);
    goff[i] = r * kRowBytes + (((lane & 15) ^ (r & 15)) * 16);
  }
  auto issue = [&](int k, char* tb, float* lb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(srows, tb + (2 * wave + i) * 1024, goff[i], k * (kTile * kRowBytes));
    if (!PASS1) {
      if (lane < 2) dma16(slse, lb + 8 * wave, 32 * wave + 16 * lane, k * kTile * 4);
    }
  };
  // the operand read of a tile: lane (n, h) takes row n's chunks 8h .. 8h+7, swizzled.  The
  // lane's eight byte offsets within a tile are computed once (and kept opaque, so they are not
  // re-derived per tile); each buffer's base then goes into the read's immediate offset.
  int roff[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    roff[s] = n * kRowBytes + (((8 * h + s) ^ (n & 15)) * 16);
    asm volatile("" : "+v"(roff[s]));
  }
  auto read_tile = [&](const char* tb, bf16x8* A) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < KS; ++s) A[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tb + roff[s]));
  };
  // s_waitcnt with vmcnt <= kPerTile, expcnt and lgkmcnt left alone (gfx9 encoding)
  constexpr int kWaitNext = (kPerTile & 15) | (7 << 4) | (15 << 8) | ((kPerTile >> 4) << 14);

  issue(0, tb0, lb0);
  issue(1, tb1, lb1);
  issue(2, tb2, lb2);
  // persistent operand straight from global memory in operand layout (rows past the end read zero)
  bf16x8 B0[KS], B1[KS];
  {
    const int64_t pbase = (PASS1 ? 0 : c0) + (int64_t)tile * PER_WG;
    const int64_t plim = PASS1 ? rows : c1;
    const int pcount = (int)(plim <= pbase ? 0 : (plim - pbase > PER_WG ? PER_WG : plim - pbase));
    const uint16_t* pg = (PASS1 ? Qg : Ig) + (pcount > 0 ? (size_t)pbase * D : 0);
    const __amdgpu_buffer_rsrc_t prs = buf_rsrc(pg, pcount * kRowBytes);
    const int r0 = (wave * kPerWave + n) * kRowBytes + h * (kRowBytes / 2);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      B0[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(prs, r0 + 16 * s, 0, 0));
      B1[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(prs, r0 + 32 * kRowBytes + 16 * s, 0, 0));
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();

  const bool live = p0 < (PASS1 ? rows : c1 - c0);   // wave-uniform
  bf16x8 A[KS];
  f32x16 cA0 = {}, cA1 = {}, cB0 = {}, cB1 = {};
  float lA[16], lB[16];
  read_tile(tb0, A);
  if (!PASS1) read_lse16(lb0, h, lA);
  if (live) mma2<D>(A, B0, B1, cA0, cA1);

  float m0, m1, s0 = 0.f, s1 = 0.f;
  if (PASS1) {
    f32x16 x0 = cA0, x1 = cA1;
    if (nt == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (s_begin + c_row(v, h) >= s_end) { x0[v] = -INFINITY; x1[v] = -INFINITY; }
    }
    m0 = fmaxf(tile_max(x0) * scale, -3.0e38f);
    m1 = fmaxf(tile_max(x1) * scale, -3.0e38f);
    m0 = fmaxf(m0, __shfl_xor(m0, 32, kWave));
    m1 = fmaxf(m1, __shfl_xor(m1, 32, kWave));
  }

  // body t: issue tile t+3 into the buffer tile t-1 used, read tile t+1, MFMAs of t+1 with the
  // epilogue of t, then wait for this wave's part of tile t+2 and meet the others
  auto body = [&](int t, char* tb_issue, float* lb_issue, const char* tb_read, const float* lb_read,
                  f32x16& cc0, f32x16& cc1, float* lc, f32x16& cn0, f32x16& cn1, float* ln) __attribute__((always_inline)) {
    issue(t + 3, tb_issue, lb_issue);
    read_tile(tb_read, A);
    if (!PASS1) read_lse16(lb_read, h, ln);
    float a0 = 0.f, a1 = 0.f;
    if (live) step_mma_epi<PASS1, D>(A, B0, B1, cn0, cn1, cc0, cc1, scale, lc, m0, m1, a0, a1);
    if (PASS1) {
      if (__builtin_expect(__ballot(!(a0 <= kRebase) || !(a1 <= kRebase)) != 0, 0)) {
        lse_fold<false>(cc0, scale, m0, s0, a0, 0, h, c1, 0, 0);
        lse_fold<false>(cc1, scale, m1, s1, a1, 0, h, c1, 0, 0);
      } else {
        s0 += a0;
        s1 += a1;
      }
    } else {
      s0 += a0;
      s1 += a1;
    }
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    __builtin_amdgcn_s_barrier();
  };
  // t % 4 fixes the buffers (issue into (t+3)%4, read (t+1)%4) and t % 2 the accumulators
  auto body_k = [&](int t, auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    char* tbs[4] = {tb0, tb1, tb2, tb3};
    float* lbs[4] = {lb0, lb1, lb2, lb3};
    if constexpr ((k & 1) != 0)
      body(t, tbs[(k + 3) & 3], lbs[(k + 3) & 3], tbs[(k + 1) & 3], lbs[(k + 1) & 3], cB0, cB1, lB, cA0, cA1, lA);
    else
      body(t, tbs[(k + 3) & 3], lbs[(k + 3) & 3], tbs[(k + 1) & 3], lbs[(k + 1) & 3], cA0, cA1, lA, cB0, cB1, lB);
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  using K3 = std::integral_constant<int, 3>;
  int t = 0;
  for (; t + 4 < nt; t += 4) {
    body_k(t, K0{});
    body_k(t + 1, K1{});
    body_k(t + 2, K2{});
    body_k(t + 3, K3{});
  }
  if (t + 1 < nt) {
    body_k(t, K0{});
    if (t + 2 < nt) {
      body_k(t + 1, K1{});
      if (t + 3 < nt) body_k(t + 2, K2{});
    }
  }
  // the last tile, nt - 1, was computed by body nt - 2 (B if that is even), or by the prologue
  const bool last_b = nt >= 2 && (nt & 1) == 0;
  f32x16* last0 = last_b ? &cB0 : &cA0;
  f32x16* last1 = last_b ? &cB1 : &cA1;
  float* llast = last_b ? lB : lA;
  if (PASS1) {
    const int64_t b0 = s_begin + (int64_t)(nt - 1) * kTile;
    lse_fold<true>(*last0, scale, m0, s0, 0.f, b0, h, s_end, 0, 0);
    lse_fold<true>(*last1, scale, m1, s1, 0.f, b0, h, s_end, 0, 0);
  } else {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      a0 += __builtin_amdgcn_exp2f(fmaf((*last0)[v], scale, -llast[v]));
      a1 += __builtin_amdgcn_exp2f(fmaf((*last1)[v], scale, -llast[v]));
    }
    s0 += a0;
    s1 += a1;
  }
  // the DMAs issued for tiles past the end must land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0);

  if (PASS1) {
    float mm = __shfl_xor(m0, 32, kWave), ss = __shfl_xor(s0, 32, kWave);
    lse_merge(m0, s0, mm, ss);
    mm = __shfl_xor(m1, 32, kWave);
    ss = __shfl_xor(s1, 32, kWave);
    lse_merge(m1, s1, mm, ss);
    if (h == 0) {
      const int64_t r0 = p0 + n, r1 = p0 + 32 + n;
      if (r0 < rows_pad) lse2[(size_t)lg * rows_pad + r0] = (r0 < rows && s0 > 0.f) ? m0 + log2f(s0) : INFINITY;
      if (r1 < rows_pad) lse2[(size_t)lg * rows_pad + r1] = (r1 < rows && s1 > 0.f) ? m1 + log2f(s1) : INFINITY;
    }
  } else {
    s0 += __shfl_xor(s0, 32, kWave);
    s1 += __shfl_xor(s1, 32, kWave);
    if (h == 0) {
      const int64_t b0 = c0 + p0 + n, b1 = c0 + p0 + 32 + n;
      if (b0 < c1) colpart[(size_t)lg * nB + b0] = s0;
      if (b1 < c1) colpart[(size_t)lg * nB + b1] = s1;
    }
  }
}

// Row lse from the pass-1 split partials, merged in split order.
__global__ __launch_bounds__(256) void meank_lse_merge(const float2* __restrict__ part1, int64_t n_rows,
                                                       int64_t rows, int64_t rows_pad, int n_split,
                                                       float* __restrict__ lse2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_rows) return;
  float m = -INFINITY, s = 0.f;
  for (int c = 0; c < n_split; ++c) {
    const float2 p = part1[(size_t)i * n_split + c];
    lse_merge(m, s, p.x, p.y);
  }
  lse2[i] = (i % rows_pad < rows && s > 0.f) ? m + log2f(s) : INFINITY;
}

// R_b = sum over (l, g) of the partials, fixed order, / LH.  A workgroup
// owns 64 columns; wave w sums lg = w, w+4, ... and the 4 waves combine in
// order.  Columns outside [c0, c1) (or, with SPAN, inside [h0, h1)) get 0.
template <bool SPAN>
__global__ __launch_bounds__(256) void meank_reduce(const float* __restrict__ colpart, int LG,
                                                    int64_t nB, int64_t c0, int64_t c1, int64_t h0,
                                                    int64_t h1, float LH, float* __restrict__ R) {
  __shared__ float part[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 64 + lane;
  const bool cand = b >= c0 && b < c1 && !(SPAN && b >= h0 && b < h1);
  float s = 0.f;
  if (cand) {
#pragma unroll 8
    for (int lg = wave; lg < LG; lg += 4) s += colpart[(size_t)lg * nB + b];
  }
  part[wave][lane] = s;
  __syncthreads();
  if (wave == 0 && b < nB)
    R[b] = cand ? (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) / LH : 0.f;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t pad32(int64_t x) { return (x + 31) / 32 * 32; }

}  // namespace

size_t kvs_meank_ws_bytes(int L, int H_q, int H_kv, int64_t Mq, int64_t nB) {
  const size_t LG = (size_t)L * H_kv;
  const int64_t rows_pad = pad32((int64_t)(H_q / H_kv) * Mq);
  return align256(LG * (size_t)rows_pad * 4) + align256(LG * (size_t)nB * 4);
}

namespace {

template <int D>
hipError_t launch_meank_score(const uint16_t* Qb, const uint16_t* Ib, int L, int H_q, int H_kv, int64_t Mq,
                              int64_t nB, int64_t c0, int64_t c1, float* R, void* ws, hipStream_t st) {
  const int LG = L * H_kv;
  const int G = H_q / H_kv;
  const int64_t rows = (int64_t)G * Mq;
  const int64_t rows_pad = pad32(rows);
  char* w = static_cast<char*>(ws);
  float* lse2 = reinterpret_cast<float*>(w);
  float* colpart = reinterpret_cast<float*>(w + align256((size_t)LG * rows_pad * 4));
  const float scale = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  if (c1 > c0 && rows > 0) {
    const int T1 = (int)ceil_div(rows_pad, kPerWG);
    const int T2 = (int)ceil_div(c1 - c0, kPerWG);
    if constexpr (D == 128) {
      hipLaunchKernelGGL((meank_pass_dma<true>), dim3((unsigned)T1 * LG), dim3(256), 0, st, Qb, Ib, LG, rows,
                         rows_pad, nB, c0, c1, T1, scale, lse2, colpart);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((meank_pass_dma<false>), dim3((unsigned)T2 * LG), dim3(256), 0, st, Qb, Ib, LG, rows,
                         rows_pad, nB, c0, c1, T2, scale, lse2, colpart);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL((meank_pass<true, false, 4, D>), dim3((unsigned)T1 * LG), dim3(256), 0, st, Qb, Ib, LG, rows,
                         rows_pad, nB, c0, c1, (int64_t)0, (int64_t)0, T1, scale, 1, lse2, nullptr, colpart);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((meank_pass<false, false, 4, D>), dim3((unsigned)T2 * LG), dim3(256), 0, st, Qb, Ib, LG, rows,
                         rows_pad, nB, c0, c1, (int64_t)0, (int64_t)0, T2, scale, 1, lse2, nullptr, colpart);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    c1 = c0;   // no candidates (or no queries): every R_b is 0
  }
  hipLaunchKernelGGL(meank_reduce<false>, dim3(ceil_div(nB, 64)), dim3(256), 0, st, colpart, LG, nB, c0, c1,
                     (int64_t)0, (int64_t)0, (float)(L * H_q), R);
  return hipGetLastError();
}

}  // namespace

hipError_t kvs_launch_meank_score(const void* Q, const void* index, int L, int H_q, int H_kv, int D,
                                  int64_t Mq, int64_t nB, int64_t c0, int64_t c1, float* R,
                                  void* ws, hipStream_t st) {
  const uint16_t* Qb = static_cast<const uint16_t*>(Q);
  const uint16_t* Ib = static_cast<const uint16_t*>(index);
  return D == 128 ? launch_meank_score<128>(Qb, Ib, L, H_q, H_kv, Mq, nB, c0, c1, R, ws, st)
                  : launch_meank_score<64>(Qb, Ib, L, H_q, H_kv, Mq, nB, c0, c1, R, ws, st);
}

// Window score (the SnapKV query window that IntentKV's Eq. 3 replaces by one
// memory vector): the same two-pass engine with the window's G*W query rows
// of each KV group in place of the Mean-K queries and the cache's keys in
// place of the block index.  Candidates are [pi, N) minus [q_s, q_e); pass 1
// is split along N so that a short window still fills the device.
namespace {

struct WindowPlan {
  int64_t rows, rows_pad, c0, c1, h0, h1;
  int T1, T2, n_split, nw1;
};

WindowPlan window_plan(int L, int H_q, int H_kv, int64_t W, int64_t N, int64_t pi, int64_t q_s, int64_t q_e) {
  WindowPlan p;
  const int LG = L * H_kv;
  p.rows = (int64_t)(H_q / H_kv) * W;
  p.rows_pad = pad32(p.rows);
  p.c0 = pi < N ? pi : N;
  p.c1 = N;
  p.h0 = q_s > p.c0 ? q_s : p.c0;
  p.h1 = q_e < N ? q_e : N;
  if (p.h1 < p.h0) p.h1 = p.h0;
  // pass 1 with two waves per workgroup when the window has at most 128 rows
  // (a 256-row workgroup would leave half its waves without rows): twice the
  // workgroups per CU, each streaming its own keys
  p.nw1 = p.rows_pad <= 2 * kPerWave ? 2 : 4;
  p.T1 = (int)ceil_div(p.rows_pad, p.nw1 * kPerWave);
  // pass 2 in two-wave workgroups too: each loads its 128 key rows and streams
  // only the few query tiles, so more, smaller workgroups overlap those phases
  // better (same-process A/B at rule-8b: 1.053-1.068 -> 1.042-1.044 ms, same bits)
  p.T2 = (int)ceil_div(p.c1 - p.c0 > 0 ? p.c1 - p.c0 : 1, 2 * kPerWave);
  // at least ~2048 workgroups in pass 1, and at least 8 tiles per split
  const int64_t want = ceil_div(2048, (int64_t)p.T1 * LG);
  const int64_t most = ceil_div(p.c1 - p.c0 > 0 ? p.c1 - p.c0 : 1, 8 * kTile);
  p.n_split = (int)(want < most ? want : most);
  if (p.n_split < 1) p.n_split = 1;
  if (p.n_split > 65535) p.n_split = 65535;
  return p;
}

}  // namespace

size_t kvs_window_ws_bytes(int L, int H_q, int H_kv, int64_t W, int64_t N) {
  const WindowPlan p = window_plan(L, H_q, H_kv, W, N, 0, 0, 0);
  const size_t LG = (size_t)L * H_kv;
  return align256(LG * (size_t)p.rows_pad * 4) + align256(LG * (size_t)p.rows_pad * p.n_split * 8) +
         align256(LG * (size_t)N * 4);
}

namespace {

template <int D>
hipError_t launch_window(const uint16_t* Qb, const uint16_t* Kb, int L, int H_q, int H_kv, int64_t W, int64_t N,
                         int64_t pi, int64_t q_s, int64_t q_e, float* score, void* ws, hipStream_t st) {
  const int LG = L * H_kv;
  WindowPlan p = window_plan(L, H_q, H_kv, W, N, pi, q_s, q_e);
  // the split count (and so the workspace) does not depend on pi or the span
  p.n_split = window_plan(L, H_q, H_kv, W, N, 0, 0, 0).n_split;
  char* w = static_cast<char*>(ws);
  float* lse2 = reinterpret_cast<float*>(w);
  w += align256((size_t)LG * p.rows_pad * 4);
  float2* part1 = reinterpret_cast<float2*>(w);
  w += align256((size_t)LG * p.rows_pad * p.n_split * 8);
  float* colpart = reinterpret_cast<float*>(w);
  const float scale = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  int64_t c0 = p.c0, c1 = p.c1;
  const bool any = c1 > c0 && !(p.h0 <= c0 && p.h1 >= c1) && p.rows > 0;
  if (any) {
    const dim3 grid1((unsigned)p.T1 * LG, (unsigned)p.n_split);
    if (p.nw1 == 2)
      hipLaunchKernelGGL((meank_pass<true, true, 2, D>), grid1, dim3(128), 0, st, Qb, Kb, LG, p.rows, p.rows_pad, N,
                         c0, c1, p.h0, p.h1, p.T1, scale, p.n_split, lse2, part1, colpart);
    else
      hipLaunchKernelGGL((meank_pass<true, true, 4, D>), grid1, dim3(256), 0, st, Qb, Kb, LG, p.rows, p.rows_pad, N,
                         c0, c1, p.h0, p.h1, p.T1, scale, p.n_split, lse2, part1, colpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.n_split > 1) {
      const int64_t n_rows = (int64_t)LG * p.rows_pad;
      hipLaunchKernelGGL(meank_lse_merge, dim3(ceil_div(n_rows, 256)), dim3(256), 0, st, part1, n_rows, p.rows,
                         p.rows_pad, p.n_split, lse2);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((meank_pass<false, true, 2, D>), dim3((unsigned)p.T2 * LG), dim3(128), 0, st, Qb, Kb, LG,
                       p.rows, p.rows_pad, N, c0, c1, p.h0, p.h1, p.T2, scale, 1, lse2, part1, colpart);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    c1 = c0;   // no candidates (or an empty window): every score is 0
  }
  hipLaunchKernelGGL(meank_reduce<true>, dim3(ceil_div(N, 64)), dim3(256), 0, st, colpart, LG, N, c0, c1, p.h0,
                     p.h1, 1.0f, score);
  return hipGetLastError();
}

}  // namespace

hipError_t kvs_launch_window(const void* K, const void* Qw, int L, int H_q, int H_kv, int D, int64_t W, int64_t N,
                             int64_t pi, int64_t q_s, int64_t q_e, float* score, void* ws, hipStream_t st) {
  const uint16_t* Qb = static_cast<const uint16_t*>(Qw);
  const uint16_t* Kb = static_cast<const uint16_t*>(K);
  return D == 128 ? launch_window<128>(Qb, Kb, L, H_q, H_kv, W, N, pi, q_s, q_e, score, ws, st)
                  : launch_window<64>(Qb, Kb, L, H_q, H_kv, W, N, pi, q_s, q_e, score, ws, st);
}
