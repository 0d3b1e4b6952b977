// Budgeted top-k with a forced set (IntentKV, Sec. 3.1, Eq. 1) and the
// slot-map redirect of the IntentKV layout layer.
//
// Scores map to order-preserving uint32 keys (sign-flip trick; NaN below every
// number; -0 -> +0), so the selection is integer-only and exact: a radix
// select over the key range [kmin, kmax] of the candidates, digits cut from the
// top of that range down, finds the threshold key T and the number of
// threshold ties k to keep; ballot/popcount ranks make the output ascending
// and hand the k ties to the lowest indices.  Up to 32768 scores one
// 1024-thread workgroup keeps every key in registers (topk_wg_kernel); above
// that, with a workspace, a few short multi-workgroup launches share the work
// (topk_mw_*); without one, one workgroup streams the scores from L2 on every
// pass (topk_stream_kernel).
#include <mutex>

#include "kvs_internal.h"

using namespace kvs;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t rank_below(uint64_t mask, int lane) {
  return (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

struct Forced {
  int f0b, f0e, f1b, f1e;
  __device__ bool operator()(int j) const { return (j >= f0b && j < f0e) || (j >= f1b && j < f1e); }
};

// The slot-map redirect of the layout layer, written by the multi-workgroup
// emit itself when asked for (out != nullptr): out[j] = kept ? in[j] : dead.
// in and out may be one array (each position is read, then written, by the
// same thread).
struct Redirect {
  const int64_t* in;
  int64_t dead;
  int64_t* out;
  __device__ __forceinline__ void operator()(int64_t j, bool keep) const {
    if (out) out[j] = keep ? in[j] : dead;
  }
};

// Keys held in registers, for n <= 4096 * V: thread t of the one 1024-thread
// workgroup owns the four consecutive positions 4 * (1024 v + t) + e (v < V,
// e < 4), read with one 16-byte load per v, so a wave's load covers 1 KB and
// the whole selection reads the scores once.  The key itself carries a
// position's class, so no per-position flags are kept: candidates take the
// order-preserving key with NaN -> 1 (below -inf, which maps to 0x007fffff), a
// forced position takes 0xffffffff (above +inf, 0xff800000) and a position
// past n takes 0.  "Kept by value" is then just key > T.
//
// The threshold key T (the C*-th largest candidate key, ties counted) and the
// number k of its ties to keep come from:
//   1. one 11-bit digit of key - min over every candidate: the top bits of the
//      candidates' own key range, so the digit spreads them over up to 2048
//      bins however narrow that range is; four LDS histograms, one per four
//      waves, then a workgroup suffix scan over the bins picks the bin holding
//      the C*-th key;
//   2. that bin's keys (at most kList of them) gathered into LDS and ranked
//      directly: T is the key with fewer than k keys above it and at least k
//      at or above it.  A bin holding more keys (a heavily tied or clustered
//      input) is resolved instead by 8-bit digits over the keys in registers,
//      one LDS histogram per wave and pass.
// The emit counts, per (v, wave), the positions kept by value and the ties
// with ballots, scans those counts in position order (v, then wave, then
// lane, then e), and writes each kept index at its final rank, so ties go to
// the lowest indices and keep_idx comes out ascending.  Loads and stores go
// through bounds-checked buffer resources: loads past n return 0, and the
// keep_idx store of an unkept position is sent out of range and dropped.
constexpr uint32_t kKeyOut = 0u, kKeyForced = 0xffffffffu;

__device__ __forceinline__ uint32_t cand_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kWgBins = 2048;      // bins of the first digit (11 bits)
constexpr int kWgHists = 4;        // first-digit histograms, one per four waves
constexpr int kList = 256;         // largest threshold bin ranked directly

template <int V>
__global__ __launch_bounds__(kThreads) void topk_wg_kernel(
    const float* __restrict__ score, int n, Forced forced, int c_star, int n_forced,
    uint8_t* __restrict__ keep_mask, int32_t* __restrict__ keep_idx, int64_t* __restrict__ n_kept) {
  // the first-digit histograms; the 8-bit passes use the same words as one
  // 256-bin histogram per wave
  __shared__ __attribute__((aligned(16))) uint32_t hist[kWgHists * kWgBins + 64];   // + one discard word per lane
  __shared__ uint32_t lst[kList];
  __shared__ uint32_t wred[kWaves][2];
  __shared__ uint32_t wsum[kWaves];
  __shared__ uint32_t state[4];             // bin or key, k still to take, bin count, list fill
  __shared__ uint32_t cnt[2][V][kWaves];    // [kept-by-value | ties][v][wave]
  static_assert(kWgHists * kWgBins >= kWaves * 256, "8-bit passes reuse the histogram words");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(score, n * 4);
  const __amdgpu_buffer_rsrc_t rm = buf_rsrc(keep_mask, n);
  const __amdgpu_buffer_rsrc_t ri = buf_rsrc(keep_idx, n * 4);

  u32x4 key[V];
#pragma unroll
  for (int v = 0; v < V; ++v)
    key[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (v * kThreads + tid), 0, 0);
  // clear the first-digit histograms while the loads are in flight
  for (int i = tid; i < kWgHists * kWgBins / 4; i += kThreads)
    reinterpret_cast<u32x4*>(hist)[i] = (u32x4){0u, 0u, 0u, 0u};
  if (tid == 0) state[3] = 0u;
  // min - 1 and max of the candidate keys: an out key (0) wraps to the top under - 1 and a
  // forced key (all ones) is below every candidate's - 1 only if there is no candidate, so
  // only the max needs the forced class masked
  uint32_t mn1 = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // the position, opaque to the compiler so that the range tests stay per-lane arithmetic
      // instead of a set of scalar bounds per (v, e)
      int p = 4 * tid + (4 * kThreads * v + e);
      asm volatile("" : "+v"(p));
      const bool in = p < n;
      const bool f = ((uint32_t)(p - forced.f0b) < (uint32_t)(forced.f0e - forced.f0b)) |
                     ((uint32_t)(p - forced.f1b) < (uint32_t)(forced.f1e - forced.f1b));
      // the candidate key, then the classes, as straight-line arithmetic (the compiler turns
      // nested selects over cand_key into two branches per position)
      const uint32_t u0 = key[v][e];
      const uint32_t u = u0 == 0x80000000u ? 0u : u0;
      const uint32_t kc0 = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      const uint32_t kc = (u & 0x7fffffffu) > 0x7f800000u ? 1u : kc0;
      const uint32_t fm = 0u - (uint32_t)f, im = 0u - (uint32_t)in;
      uint32_t kk = ((kc & ~fm) | fm) & im;
      mn1 = min(mn1, kk - 1u);
      mx = max(mx, kk == kKeyForced ? 0u : kk);
      // opaque from here on: the compiler would otherwise keep kk - 1 of every position live, a
      // second array, to reuse in the candidate tests of the later passes
      asm volatile("" : "+v"(kk));
      key[v][e] = kk;
    }
    // and the running min and max are materialised here, so they are not regrouped into one
    // tree over every position at the end (which kept each position's kk live until then)
    asm volatile("" : "+v"(mn1), "+v"(mx));
  }
  auto is_cand = [&](uint32_t k) -> bool { return (k != kKeyOut) & (k != kKeyForced); };
  // Marks the keys as rewritten (no instruction): each phase then computes its own compares
  // instead of the compiler keeping one phase's compare masks live for the next, spilled.
  auto fresh_keys = [&]() {
#pragma unroll
    for (int v = 0; v < V; ++v)
      asm volatile("" : "+v"(key[v][0]), "+v"(key[v][1]), "+v"(key[v][2]), "+v"(key[v][3]));
  };

  // C <= |F| (c_star == 0) keeps the forced set only: T = 0xfffffffe.
  uint32_t kT = 0xfffffffeu, k_tie = 0;
  if (c_star > 0) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn1 = min(mn1, (uint32_t)__shfl_xor((int)mn1, o, kWave));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
    }
    if (lane == 0) { wred[wave][0] = mn1; wred[wave][1] = mx; }
    __syncthreads();
    {
      // lane w < 16 takes wave w's pair; a 16-lane butterfly combines them (one pair of loads per
      // lane rather than all 32 words in every lane's registers)
      uint32_t a = lane < kWaves ? wred[lane][0] : 0xffffffffu, b = lane < kWaves ? wred[lane][1] : 0u;
#pragma unroll
      for (int o = kWaves / 2; o > 0; o >>= 1) {
        a = min(a, (uint32_t)__shfl_xor((int)a, o, kWave));
        b = max(b, (uint32_t)__shfl_xor((int)b, o, kWave));
      }
      mn1 = (uint32_t)__builtin_amdgcn_readlane((int)a, 0);
      mx = (uint32_t)__builtin_amdgcn_readlane((int)b, 0);
    }
    const uint32_t mn = mn1 + 1u;   // there is a candidate: c_star < n - |F|
    const uint32_t range = mx - mn;
    const int bits = range ? 32 - __clz(range) : 0;
    uint32_t prefix = 0u, k = (uint32_t)c_star;
    int rem = bits;   // low bits of key - mn not yet fixed by prefix
    if (bits > 0) {
      // 1. first digit: the top wd bits of key - mn (all of them when the range is narrow)
      const int wd = min(11, bits), sh = bits - wd;
      {
        // every position adds: a forced or out position to its lane's discard word, so the loop has
        // no branch (a branch per position kept a compare mask per position live in scalar registers)
        const uint32_t h = (uint32_t)(wave & (kWgHists - 1)) * kWgBins, discard = kWgHists * kWgBins + lane;
        uint32_t mnp = mn;
        asm volatile("" : "+v"(mnp));   // keep key - mn from being hoisted into a second key array
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            atomicAdd(hist + (is_cand(key[v][e]) ? h + ((key[v][e] - mnp) >> sh) : discard), 1u);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      // thread t sums bins 2t and 2t+1 over the histograms; suffix sums from the top bin down
      const int b0 = 2 * tid;
      uint32_t c0 = 0u, c1 = 0u;
#pragma unroll
      for (int q = 0; q < kWgHists; ++q) { c0 += hist[q * kWgBins + b0]; c1 += hist[q * kWgBins + b0 + 1]; }
      uint32_t incl = c0 + c1;   // inclusive suffix sum over the lanes (bins >= 2t within the wave)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_down((int)incl, o, kWave);
        if (lane + o < 64) incl += t;
      }
      if (lane == 0) wsum[wave] = incl;
      __syncthreads();
      uint32_t above = lane < kWaves && lane > wave ? wsum[lane] : 0u;   // bins of the later waves
#pragma unroll
      for (int o = kWaves / 2; o > 0; o >>= 1) above += (uint32_t)__shfl_xor((int)above, o, kWave);
      above = (uint32_t)__builtin_amdgcn_readlane((int)above, 0);
      const uint32_t s_lo = incl + above;   // bins >= 2t
      const uint32_t s_hi = s_lo - c0;      // bins >= 2t + 1
      const uint32_t s_up = s_hi - c1;      // bins >= 2t + 2
      if (s_up < k && k <= s_hi) { state[0] = b0 + 1; state[1] = k - s_up; state[2] = c1; }
      if (s_hi < k && k <= s_lo) { state[0] = b0; state[1] = k - s_hi; state[2] = c0; }
      __syncthreads();
      prefix = state[0];
      k = state[1];
      const uint32_t m = state[2];
      rem = sh;
      fresh_keys();
      if (rem > 0 && m <= (uint32_t)kList) {
        // 2. gather the bin's keys and rank them directly
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (is_cand(key[v][e]) && ((key[v][e] - mn) >> sh) == prefix) lst[atomicAdd(&state[3], 1u)] = key[v][e];
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        if ((uint32_t)tid < m) {
          const uint32_t x = lst[tid];
          uint32_t gt = 0u, eq = 0u;
          for (uint32_t i = 0; i < m; ++i) {
            const uint32_t y = lst[i];
            gt += y > x;
            eq += y == x;
          }
          // every thread holding the threshold key writes the same two words
          if (gt < k && k <= gt + eq) { state[0] = x; state[1] = k - gt; }
        }
        __syncthreads();
        kT = state[0];
        k_tie = state[1];
        rem = -1;   // resolved
      }
    }
    if (rem >= 0) {
      // the bin is resolved by 8-bit digits over the keys in registers (rem
      // may be 0: the bin, or the whole range, is one key value)
      uint32_t* h = hist + wave * 256;
      for (int p = 0; 8 * p < rem; ++p) {
        fresh_keys();
        const int sh2 = max(rem - 8 * (p + 1), 0), wd2 = rem - 8 * p - sh2;
        for (int i = lane; i < 256; i += 64) h[i] = 0u;
        uint32_t mnp = mn;
        asm volatile("" : "+v"(mnp));
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t rel = key[v][e] - mnp;
            const uint32_t hi = (uint32_t)((uint64_t)rel >> (sh2 + wd2));
            if (is_cand(key[v][e]) & (hi == prefix)) atomicAdd(h + ((rel >> sh2) & ((1u << wd2) - 1u)), 1u);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        if (wave == 0) {
          uint32_t c[4] = {0u, 0u, 0u, 0u};
          for (int w = 0; w < kWaves; ++w) {
            const u32x4 hv = *reinterpret_cast<const u32x4*>(hist + w * 256 + 4 * lane);
            c[0] += hv[0]; c[1] += hv[1]; c[2] += hv[2]; c[3] += hv[3];
          }
          const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
          uint32_t incl = lsum;   // candidates in bins >= 4*lane
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = (uint32_t)__shfl_down((int)incl, o, kWave);
            if (lane + o < 64) incl += t;
          }
          const uint32_t above = incl - lsum;
          if (above < k && k <= incl) {
            uint32_t a = above;
            for (int i = 3; i >= 0; --i) {
              if (a + c[i] >= k) {
                state[0] = (prefix << wd2) | (uint32_t)(4 * lane + i);
                state[1] = k - a;
                break;
              }
              a += c[i];
            }
          }
        }
        __syncthreads();   // wave 0 has read every histogram before the next pass clears them
        prefix = state[0];
        k = state[1];
      }
      kT = mn + prefix;
      k_tie = k;
    }
  }

  // Emit.  Counts per (v, wave) of positions kept by value and of ties, written by lane 0 as
  // each v is counted (so only one v's ballots are live at a time).
  fresh_keys();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    uint32_t nd = 0u, nt = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nd += (uint32_t)__popcll(__ballot(key[v][e] > kT));
      nt += (uint32_t)__popcll(__ballot(key[v][e] == kT));
    }
    if (lane == 0) { cnt[0][v][wave] = nd; cnt[1][v][wave] = nt; }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if (wave < 2) {
    // exclusive prefix over the V * 16 (v, wave) counts in position order;
    // wave 0 takes the kept-by-value counts, wave 1 the ties
    constexpr int E = V * kWaves, PER = (E + 63) / 64;
    uint32_t* c = &cnt[wave][0][0];
    uint32_t a[PER];
    uint32_t s = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ix = lane * PER + i;
      a[i] = ix < E ? c[ix] : 0u;
      s += a[i];
    }
    uint32_t incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_up((int)incl, o, kWave);
      if (lane >= o) incl += t;
    }
    uint32_t run = incl - s;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ix = lane * PER + i;
      if (ix < E) c[ix] = run;
      run += a[i];
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  // the threshold again, opaque to the compiler: otherwise it keeps every compare mask of the
  // counting loop live (in spilled scalar registers) to reuse them here
  asm volatile("" : "+v"(kT));
  // and the positions too, or it keeps the classification's position of every (v, e) live
  int tq = tid;
  asm volatile("" : "+v"(tq));
  fresh_keys();
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int q = v * kThreads + tq;    // the lane's positions are 4q .. 4q + 3
    uint32_t def_before = cnt[0][v][wave], tie_before = cnt[1][v][wave];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      def_before += (uint32_t)__popcll(__ballot(key[v][e] > kT) & below);
      tie_before += (uint32_t)__popcll(__ballot(key[v][e] == kT) & below);
    }
    uint32_t mask = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool gt = key[v][e] > kT, eq = key[v][e] == kT;
      const bool keep = gt | (eq & (tie_before < k_tie));
      const uint32_t r = def_before + min(tie_before, k_tie);
      buf_store4((uint32_t)(4 * q + e), ri, keep ? (int)(4 * r) : 0x7fffffff);
      mask |= (keep ? 1u : 0u) << (8 * e);
      def_before += gt;
      tie_before += eq;
    }
    if (4 * q + 3 < n) {
      buf_store4(mask, rm, 4 * q);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_store1((uint8_t)(mask >> (8 * e)), rm, 4 * q + e < n ? 4 * q + e : 0x7fffffff);
    }
    __builtin_amdgcn_sched_barrier(0);   // one v at a time: bounded register use
  }
  if (tid == 0) *n_kept = (int64_t)n_forced + c_star;
}

// Inputs too large to keep in registers: every pass streams the scores from
// global memory (L2-resident after the first) in batches of kStreamU keys
// per thread, all of a batch's loads in flight together, with the same key
// classes, top-aligned digits and double-buffered histograms as above.  The
// emit pass ranks one batch at a time: per-(key slot, wave) counts scanned in
// position order within the batch, on top of running totals of the batches
// before it.
constexpr int kStreamU = 16;

__global__ __launch_bounds__(kThreads) void topk_stream_kernel(
    const float* __restrict__ score, int n, Forced forced, int c_star, int n_forced,
    uint8_t* __restrict__ keep_mask, int32_t* __restrict__ keep_idx, int64_t* __restrict__ n_kept) {
  constexpr int U = kStreamU;
  __shared__ uint32_t hist[2][kWaves][256];
  __shared__ uint32_t wred[kWaves][2];
  __shared__ uint32_t state[2];
  __shared__ uint32_t cnt[2][U][kWaves];   // [kept-by-value | ties][u][wave] of the current batch
  __shared__ uint32_t ubase[2][U];
  __shared__ uint32_t btotal[2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int kBatch = kThreads * U;

  // keys of positions b0 + 1024u + tid, u < U, classed as in topk_wg_kernel
  // (positions in 64 bits: a batch may reach past 2^31 - 1)
  auto load_keys = [&](int64_t b0, uint32_t* key) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = score[min(b0 + u * kThreads + tid, (int64_t)n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = b0 + u * kThreads + tid;
      key[u] = j >= n ? kKeyOut : (forced((int)j) ? kKeyForced : cand_key(v[u]));
    }
  };
  auto is_cand = [](uint32_t k) -> bool { return (k != kKeyOut) & (k != kKeyForced); };

  uint32_t kT = 0xfffffffeu, k_tie = 0;   // c_star == 0 keeps the forced set only
  if (c_star > 0) {
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0][0])[i] = 0u;
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int64_t b0 = 0; b0 < n; b0 += kBatch) {
      uint32_t key[U];
      load_keys(b0, key);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool c = is_cand(key[u]);
        mn = min(mn, c ? key[u] : 0xffffffffu);
        mx = max(mx, c ? key[u] : 0u);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
      mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
    }
    if (lane == 0) { wred[wave][0] = mn; wred[wave][1] = mx; }
    __syncthreads();
    mn = wred[0][0]; mx = wred[0][1];
    for (int w = 1; w < kWaves; ++w) { mn = min(mn, wred[w][0]); mx = max(mx, wred[w][1]); }
    const uint32_t range = mx - mn;
    const int bits = range ? 32 - __clz(range) : 0;
    const int ndig = (bits + 7) / 8;
    uint32_t prefix = 0, k = (uint32_t)c_star;
    int buf = 0;
    for (int p = 0; p < ndig; ++p) {
      const int sh = max(bits - 8 * (p + 1), 0), wd = bits - 8 * p - sh;
      uint32_t* h = &hist[buf][wave][0];
      for (int64_t b0 = 0; b0 < n; b0 += kBatch) {
        uint32_t key[U];
        load_keys(b0, key);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t rel = key[u] - mn;
          const uint32_t hi = (uint32_t)((uint64_t)rel >> (sh + wd));
          if (is_cand(key[u]) & (hi == prefix)) atomicAdd(h + ((rel >> sh) & ((1u << wd) - 1u)), 1u);
        }
      }
      for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[buf ^ 1][0][0])[i] = 0u;
      __syncthreads();
      if (wave == 0) {
        uint32_t c[4] = {0u, 0u, 0u, 0u};
        for (int w = 0; w < kWaves; ++w) {
          const u32x4 hv = *reinterpret_cast<const u32x4*>(&hist[buf][w][4 * lane]);
          c[0] += hv[0]; c[1] += hv[1]; c[2] += hv[2]; c[3] += hv[3];
        }
        const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
        uint32_t incl = lsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = (uint32_t)__shfl_down((int)incl, o, kWave);
          if (lane + o < 64) incl += t;
        }
        const uint32_t above = incl - lsum;
        if (above < k && k <= incl) {
          uint32_t a = above;
          for (int i = 3; i >= 0; --i) {
            if (a + c[i] >= k) {
              state[0] = (prefix << wd) | (uint32_t)(4 * lane + i);
              state[1] = k - a;
              break;
            }
            a += c[i];
          }
        }
      }
      __syncthreads();
      prefix = state[0];
      k = state[1];
      buf ^= 1;
    }
    kT = mn + prefix;
    k_tie = k;
  }

  // Emit, one batch at a time, ranks continuing from the batches before.
  uint32_t run_def = 0, run_tie = 0;
  for (int64_t b0 = 0; b0 < n; b0 += kBatch) {
    uint32_t key[U];
    load_keys(b0, key);
    uint32_t cv0 = 0u, cv1 = 0u;                 // lane u: this wave's counts of key slot u
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t nd = (uint32_t)__popcll(__ballot(key[u] > kT));
      const uint32_t nt = (uint32_t)__popcll(__ballot(key[u] == kT));
      if (lane == u) { cv0 = nd; cv1 = nt; }
    }
    if (lane < U) { cnt[0][lane][wave] = cv0; cnt[1][lane][wave] = cv1; }
    __syncthreads();
    if (tid < 2 * U) {
      const int which = tid / U, u = tid - which * U;
      uint32_t run = 0;
      for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = cnt[which][u][w];
        cnt[which][u][w] = run;
        run += c;
      }
      ubase[which][u] = run;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const uint32_t a = lane < U ? ubase[which][lane] : 0u;
        uint32_t incl = a;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = (uint32_t)__shfl_up((int)incl, o, kWave);
          if (lane >= o) incl += t;
        }
        if (lane < U) ubase[which][lane] = incl - a;
        if (lane == 63) btotal[which] = incl;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = b0 + u * kThreads + tid;
      const bool tie = key[u] == kT;
      const uint64_t bt = __ballot(tie);
      const uint32_t def_before = run_def + ubase[0][u] + cnt[0][u][wave];
      const uint32_t tie_before = run_tie + ubase[1][u] + cnt[1][u][wave];
      const bool keep = (key[u] > kT) | (tie & (tie_before + rank_below(bt, lane) < k_tie));
      const uint64_t bk = __ballot(keep);
      if (j < n) keep_mask[j] = keep ? 1 : 0;
      if (keep) keep_idx[def_before + min(tie_before, k_tie) + rank_below(bk, lane)] = (int32_t)j;
    }
    run_def += btotal[0];
    run_tie += btotal[1];
    __syncthreads();   // the next batch rewrites cnt, ubase and btotal
  }
  if (tid == 0) *n_kept = (int64_t)n_forced + c_star;
}

// Multi-workgroup selection for n > 32768: one workgroup of 256 threads per
// 2048-position slice, each thread holding 8 classed keys, and a few short
// launches instead of one workgroup's long passes (whose LDS-atomic
// histograms over every key are what limits them).  State lives in the
// workspace: candidate key min/max, the radix prefix and the count k still to
// place, an arrival ticket, a 256-bin histogram and per-slice counts.
//   topk_mw_init     state <- (min = ~0, max = 0, prefix 0, k = C*), histogram 0
//   topk_mw_minmax   per-slice min/max of the candidate keys -> atomicMin/Max
//   topk_mw_pass<p>  digit p of the range, top-aligned: each slice adds its
//                    histogram of the prefix-matching keys with integer atomics
//                    (sums independent of order); the last slice to arrive
//                    picks the bin, advances prefix and k, clears the histogram
//   topk_mw_count    per-slice counts of kept-by-value and tie positions
//   topk_mw_emit     each slice ranks its positions from the counts before it
constexpr int kMwThreads = 256;
constexpr int kMwKeys = 8;                          // keys per thread
constexpr int kMwSlice = kMwThreads * kMwKeys;      // positions per workgroup
constexpr int kMwWaves = kMwThreads / 64;
enum { kMwMin = 0, kMwMax, kMwPrefix, kMwK, kMwTicket, kMwHist = 16, kMwCounts = kMwHist + 256 };

struct MwArgs {
  const float* score;
  int n;
  Forced forced;
  int c_star;
  uint32_t* ws;
};

// Keys of positions slice0 + 256u + tid, classed as in topk_wg_kernel.
__device__ __forceinline__ void mw_keys(const MwArgs& a, uint32_t* key) {
  const int64_t slice0 = (int64_t)blockIdx.x * kMwSlice;
  float v[kMwKeys];
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) v[u] = a.score[min(slice0 + u * kMwThreads + threadIdx.x, (int64_t)a.n - 1)];
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    const int64_t j = slice0 + u * kMwThreads + threadIdx.x;
    key[u] = j >= a.n ? kKeyOut : (a.forced((int)j) ? kKeyForced : cand_key(v[u]));
  }
}
__device__ __forceinline__ bool mw_cand(uint32_t k) { return (k != kKeyOut) & (k != kKeyForced); }

__device__ __forceinline__ uint32_t mw_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_init(MwArgs a, int64_t n_kept_value, int64_t* n_kept) {
  uint32_t* ws = a.ws;
  const int t = threadIdx.x;
  if (t == 0) {
    ws[kMwMin] = 0xffffffffu;
    ws[kMwMax] = 0u;
    ws[kMwPrefix] = 0u;
    ws[kMwK] = (uint32_t)a.c_star;
    ws[kMwTicket] = 0u;
    *n_kept = n_kept_value;
  }
  ws[kMwHist + t] = 0u;
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_minmax(MwArgs a) {
  uint32_t key[kMwKeys];
  mw_keys(a, key);
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    const bool c = mw_cand(key[u]);
    mn = min(mn, c ? key[u] : 0xffffffffu);
    mx = max(mx, c ? key[u] : 0u);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
  }
  if ((threadIdx.x & 63) == 0) {
    if (mn != 0xffffffffu) atomicMin(a.ws + kMwMin, mn);
    if (mx != 0u) atomicMax(a.ws + kMwMax, mx);
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_pass(MwArgs a, int p) {
  __shared__ uint32_t hist[kMwWaves][256];
  __shared__ uint32_t s_last;
  uint32_t* ws = a.ws;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const uint32_t mn = mw_load(ws + kMwMin), mx = mw_load(ws + kMwMax);
  const uint32_t range = mx - mn;
  const int bits = range ? 32 - __clz(range) : 0;
  if (p >= (bits + 7) / 8) return;                   // every workgroup alike: this digit does not exist
  const int sh = max(bits - 8 * (p + 1), 0), wd = bits - 8 * p - sh;
  const uint32_t prefix = mw_load(ws + kMwPrefix);
  for (int i = t; i < kMwWaves * 256; i += kMwThreads) (&hist[0][0])[i] = 0u;
  uint32_t key[kMwKeys];
  mw_keys(a, key);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    const uint32_t rel = key[u] - mn;
    const uint32_t hi = (uint32_t)((uint64_t)rel >> (sh + wd));
    if (mw_cand(key[u]) & (hi == prefix)) atomicAdd(&hist[wave][(rel >> sh) & ((1u << wd) - 1u)], 1u);
  }
  __syncthreads();
  {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kMwWaves; ++w) c += hist[w][t];
    if (c) atomicAdd(ws + kMwHist + t, c);
  }
  __threadfence();                                   // the bins are added before this slice arrives
  __syncthreads();
  if (t == 0) s_last = atomicAdd(ws + kMwTicket, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (wave == 0) {
    // suffix scan over the 256 bins: lane l holds bins 4l..4l+3
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = mw_load(ws + kMwHist + 4 * lane + i);
    const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = lsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = (uint32_t)__shfl_down((int)incl, o, kWave);
      if (lane + o < 64) incl += v;
    }
    const uint32_t above = incl - lsum;
    const uint32_t k = mw_load(ws + kMwK);
    if (above < k && k <= incl) {
      uint32_t acc = above;
      for (int i = 3; i >= 0; --i) {
        if (acc + c[i] >= k) {
          ws[kMwPrefix] = (prefix << wd) | (uint32_t)(4 * lane + i);
          ws[kMwK] = k - acc;
          break;
        }
        acc += c[i];
      }
    }
  }
  __syncthreads();                                   // wave 0 has read every bin before any is cleared
  ws[kMwHist + t] = 0u;                              // clean for the next digit
  if (t == 0) ws[kMwTicket] = 0u;
}

// threshold key T and ties to keep, from the state the passes left
__device__ __forceinline__ void mw_threshold(const MwArgs& a, uint32_t& kT, uint32_t& k_tie) {
  if (a.c_star == 0) { kT = 0xfffffffeu; k_tie = 0u; return; }
  kT = mw_load(a.ws + kMwMin) + mw_load(a.ws + kMwPrefix);
  k_tie = mw_load(a.ws + kMwK);
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_count(MwArgs a) {
  __shared__ uint32_t part[kMwWaves][2];
  uint32_t kT, k_tie;
  mw_threshold(a, kT, k_tie);
  uint32_t key[kMwKeys];
  mw_keys(a, key);
  uint32_t nd = 0, nt = 0;
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    nd += (uint32_t)__popcll(__ballot(key[u] > kT));
    nt += (uint32_t)__popcll(__ballot(key[u] == kT));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { part[wave][0] = nd; part[wave][1] = nt; }
  __syncthreads();
  if (threadIdx.x < 2) {
    uint32_t c = 0;
    for (int w = 0; w < kMwWaves; ++w) c += part[w][threadIdx.x];
    a.ws[kMwCounts + 2 * blockIdx.x + threadIdx.x] = c;
  }
}

__global__ __launch_bounds__(kMwThreads) void topk_mw_emit(MwArgs a, uint8_t* __restrict__ keep_mask,
                                                           int32_t* __restrict__ keep_idx, Redirect rd) {
  __shared__ uint32_t cnt[2][kMwKeys][kMwWaves];
  __shared__ uint32_t base[2];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t slice0 = (int64_t)blockIdx.x * kMwSlice;
  // the slots to redirect, fetched before anything waits
  int64_t sv[kMwKeys];
  if (rd.out) {
#pragma unroll
    for (int u = 0; u < kMwKeys; ++u) sv[u] = rd.in[min(slice0 + u * kMwThreads + t, (int64_t)a.n - 1)];
  }
  uint32_t kT, k_tie;
  mw_threshold(a, kT, k_tie);
  uint32_t key[kMwKeys];
  mw_keys(a, key);
  // counts of the slices before this one, summed in slice order by wave 0
  if (wave == 0) {
    uint32_t d = 0, e = 0;
    for (int w = lane; w < (int)blockIdx.x; w += 64) {
      d += a.ws[kMwCounts + 2 * w];
      e += a.ws[kMwCounts + 2 * w + 1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      d += (uint32_t)__shfl_xor((int)d, o, kWave);
      e += (uint32_t)__shfl_xor((int)e, o, kWave);
    }
    if (lane == 0) { base[0] = d; base[1] = e; }
  }
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    const uint32_t nd = (uint32_t)__popcll(__ballot(key[u] > kT));
    const uint32_t nt = (uint32_t)__popcll(__ballot(key[u] == kT));
    if (lane == 0) { cnt[0][u][wave] = nd; cnt[1][u][wave] = nt; }
  }
  __syncthreads();
  if (t < 2) {                                       // exclusive prefix over (u, wave) in position order
    uint32_t run = base[t];
    for (int u = 0; u < kMwKeys; ++u)
      for (int w = 0; w < kMwWaves; ++w) {
        const uint32_t c = cnt[t][u][w];
        cnt[t][u][w] = run;
        run += c;
      }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMwKeys; ++u) {
    const int64_t j = slice0 + u * kMwThreads + t;
    const bool tie = key[u] == kT;
    const uint64_t bt = __ballot(tie);
    const uint32_t def_before = cnt[0][u][wave], tie_before = cnt[1][u][wave];
    const bool keep = (key[u] > kT) | (tie & (tie_before + rank_below(bt, lane) < k_tie));
    const uint64_t bk = __ballot(keep);
    if (j < a.n) {
      keep_mask[j] = keep ? 1 : 0;
      if (rd.out) rd.out[j] = keep ? sv[u] : rd.dead;
    }
    if (keep) keep_idx[def_before + min(tie_before, k_tie) + rank_below(bk, lane)] = (int32_t)j;
  }
}

// C* >= |H|: everything is kept.
__global__ __launch_bounds__(256) void keep_all_kernel(int n, uint8_t* __restrict__ keep_mask,
                                                       int32_t* __restrict__ keep_idx,
                                                       int64_t* __restrict__ n_kept, Redirect rd) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < n) {
    keep_mask[j] = 1;
    keep_idx[j] = j;
    rd(j, true);
  }
  if (j == 0) *n_kept = n;
}

__global__ __launch_bounds__(256) void slotmap_kernel(const int64_t* __restrict__ in,
                                                      const uint8_t* __restrict__ mask, int64_t N,
                                                      int64_t dead, int64_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < N; j += stride)
    out[j] = mask[j] ? in[j] : dead;
}

}  // namespace

// Up to kWgMaxN scores one workgroup holds every key in registers and needs
// no workspace; above that the multi-workgroup path keeps state words, a
// histogram and two counts per 2048-position slice.  (The one workgroup also
// fits 98304 keys, 96 per thread, but one CU reads the scores at ~25 GB/s:
// at n = 92160 its load alone took 15 us, and the call as long as the
// multi-workgroup path's eight short launches.)
constexpr int64_t kWgMaxN = 8 * 4 * kThreads;

size_t kvs_topk_ws_bytes(int64_t n) {
  if (n <= kWgMaxN) return 0;
  const int64_t slices = (n + kMwSlice - 1) / kMwSlice;
  return (size_t)(kMwCounts + 2 * slices) * 4;
}

hipError_t kvs_launch_topk(const float* score, int64_t n, int64_t f0b, int64_t f0e, int64_t f1b,
                           int64_t f1e, int64_t n_forced, int64_t c_star, uint8_t* keep_mask,
                           int32_t* keep_idx, int64_t* n_kept, void* ws, hipStream_t st,
                           const int64_t* slot_in, int64_t dead_slot, int64_t* slot_out) {
  const Redirect rd{slot_in, dead_slot, slot_out};
  if (c_star >= n - n_forced) {   // includes n == 0: still writes n_kept
    const unsigned blocks = n > 0 ? ceil_div(n, 256) : 1u;
    hipLaunchKernelGGL(keep_all_kernel, dim3(blocks), dim3(256), 0, st, (int)n, keep_mask, keep_idx,
                       n_kept, rd);
    return hipGetLastError();
  }
  Forced f{(int)f0b, (int)f0e, (int)f1b, (int)f1e};
  // One workgroup selects up to kWgMaxN scores (or more without a workspace, streaming them); its
  // slot traffic would queue behind that one workgroup, so the redirect runs as its own kernel after
  // it.  The multi-workgroup emit writes it itself.
#define TOPK_WG(V)                                                                                \
  hipLaunchKernelGGL(topk_wg_kernel<V>, dim3(1), dim3(kThreads), 0, st, score, (int)n, f, (int)c_star, \
                     (int)n_forced, keep_mask, keep_idx, n_kept)
  if (n <= kWgMaxN || ws == nullptr) {
    if (n <= 2 * 4 * kThreads) TOPK_WG(2);
    else if (n <= kWgMaxN) TOPK_WG(8);
    else
      hipLaunchKernelGGL(topk_stream_kernel, dim3(1), dim3(kThreads), 0, st, score, (int)n, f,
                         (int)c_star, (int)n_forced, keep_mask, keep_idx, n_kept);
    if (slot_out != nullptr) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return kvs_launch_slotmap(slot_in, keep_mask, n, dead_slot, slot_out, st);
    }
  }
#undef TOPK_WG
  else {
    MwArgs a{score, (int)n, f, (int)c_star, static_cast<uint32_t*>(ws)};
    const dim3 grid((unsigned)((n + kMwSlice - 1) / kMwSlice)), block(kMwThreads);
    hipLaunchKernelGGL(topk_mw_init, dim3(1), block, 0, st, a, (int64_t)n_forced + c_star, n_kept);
    if (c_star > 0) {
      hipLaunchKernelGGL(topk_mw_minmax, grid, block, 0, st, a);
      for (int p = 0; p < 4; ++p) hipLaunchKernelGGL(topk_mw_pass, grid, block, 0, st, a, p);
    }
    hipLaunchKernelGGL(topk_mw_count, grid, block, 0, st, a);
    hipLaunchKernelGGL(topk_mw_emit, grid, block, 0, st, a, keep_mask, keep_idx, rd);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k that allocates nothing, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid it).  The
// multi-workgroup selection keeps its state (key range, radix prefix, arrival
// ticket, histogram, per-slice counts) in `scratch`, a file-scope device
// array sized for kvs_topk_noalloc_max_n() scores, instead of a caller
// workspace.  Each device holds its own copy at its own address from the
// first call on that device until the process ends, and every call on a
// device shares it: calls that overlap on one device race.  Nothing carries
// over between calls -- topk_mw_init rewrites every state word the later
// kernels read, and each slice writes its counts before any slice reads them.
constexpr int64_t kNoAllocMaxN = (int64_t)1 << 24;
constexpr int kNoAllocWords = kMwCounts + 2 * (int)((kNoAllocMaxN + kMwSlice - 1) / kMwSlice);

static __device__ __align__(256) uint32_t scratch[kNoAllocWords];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once resolved

// Device address of `scratch` on the device that runs stream st.  In host code
// the array's name is only a host-side handle: the address the kernels take
// comes from hipGetSymbolAddress, resolved once per device with that device
// current, and kept.
hipError_t scratch_for(hipStream_t st, uint32_t** out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (st != nullptr) {
    e = hipStreamGetDevice(st, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

int64_t kvs_topk_noalloc_max_n() { return kNoAllocMaxN; }

hipError_t kvs_launch_topk_noalloc(const float* score, int64_t n, int64_t f0b, int64_t f0e, int64_t f1b,
                                   int64_t f1e, int64_t n_forced, int64_t c_star, uint8_t* keep_mask,
                                   int32_t* keep_idx, int64_t* n_kept, hipStream_t st) {
  uint32_t* ws = nullptr;
  if (kvs_topk_ws_bytes(n) > 0) {                     // the multi-workgroup path needs the state
    if (kvs_topk_ws_bytes(n) > sizeof(scratch)) return hipErrorInvalidValue;
    const hipError_t e = scratch_for(st, &ws);
    if (e != hipSuccess) return e;
  }
  return kvs_launch_topk(score, n, f0b, f0e, f1b, f1e, n_forced, c_star, keep_mask, keep_idx, n_kept, ws, st,
                         nullptr, 0, nullptr);
}

hipError_t kvs_launch_slotmap(const int64_t* in, const uint8_t* mask, int64_t N, int64_t dead,
                              int64_t* out, hipStream_t st) {
  if (N == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((N + 255) / 256 < 4096 ? (N + 255) / 256 : 4096);
  hipLaunchKernelGGL(slotmap_kernel, dim3(blocks), dim3(256), 0, st, in, mask, N, dead, out);
  return hipGetLastError();
}
