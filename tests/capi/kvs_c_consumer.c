/*
 * A plain C consumer of the library: device memory from hipMalloc, no PyTorch, every step through
 * the C ABI of kvs.h.  It runs an IntentKV rule turn (QueryMemory over three turns, rule score,
 * top-k with the forced set, slot redirect, both also fused in one call) and a KVMEM Mean-K step (index build, R_b, sink/recent
 * + budget selection, re-RoPE scatter through a page table) on seeded synthetic inputs and checks
 * what holds exactly: unit-norm memory rows, sum(rule) = L*H_q, zeros on the forced sets, the
 * selection sizes, ascending valid top-C* selections of the scores returned, the slot map, the
 * index of a block against its mean, sum(R) = Mq, V pages copied bit for bit, K pair norms kept by
 * the rotation, the no-allocation and the fused top-k equal to the workspace one, and identical
 * bits on a second run.  Exit status = number of failed checks.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvs.h"

static int failures = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, "FAIL %d: ", __LINE__); \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, "\n");                  \
      ++failures;                             \
    }                                         \
  } while (0)
#define HIP(x)                                                                 \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "HIP error %s at %d\n", hipGetErrorString(e_), __LINE__); \
      exit(100);                                                               \
    }                                                                          \
  } while (0)
#define KVS(x)                                                                        \
  do {                                                                                \
    kvs_status s_ = (x);                                                              \
    if (s_ != KVS_OK) {                                                               \
      fprintf(stderr, "kvs error %s at %d\n", kvs_status_string(s_), __LINE__);        \
      exit(101);                                                                      \
    }                                                                                 \
  } while (0)

/* splitmix64 -> uniform in [-1, 1) */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static uint16_t to_bf16(float f) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static void* dalloc(size_t bytes) {
  void* p = NULL;
  HIP(hipMalloc(&p, bytes > 0 ? bytes : 1));
  return p;
}
static void up(void* d, const void* h, size_t n) { HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice)); }
static void down(void* h, const void* d, size_t n) { HIP(hipMemcpy(h, d, n, hipMemcpyDeviceToHost)); }

/* n_kept, ascending, forced kept, and no dropped candidate above a kept one */
static void check_selection(const float* score, int64_t n, int64_t f0b, int64_t f0e, int64_t f1b, int64_t f1e,
                            int64_t C, const uint8_t* keep, const int32_t* idx, int64_t nk, const char* what) {
  int64_t forced = 0;
  for (int64_t j = 0; j < n; ++j) forced += (j >= f0b && j < f0e) || (j >= f1b && j < f1e);
  const int64_t want = forced + (C > forced ? (C - forced < n - forced ? C - forced : n - forced) : 0);
  CHECK(nk == want, "%s: n_kept %lld want %lld", what, (long long)nk, (long long)want);
  float kept_min = INFINITY, dropped_max = -INFINITY;
  int64_t count = 0;
  for (int64_t j = 0; j < n; ++j) {
    const int f = (j >= f0b && j < f0e) || (j >= f1b && j < f1e);
    if (f) CHECK(keep[j] == 1, "%s: forced position %lld dropped", what, (long long)j);
    count += keep[j];
    if (!f && keep[j] && score[j] < kept_min) kept_min = score[j];
    if (!f && !keep[j] && score[j] > dropped_max) dropped_max = score[j];
  }
  CHECK(count == nk, "%s: mask holds %lld, n_kept %lld", what, (long long)count, (long long)nk);
  for (int64_t r = 1; r < nk; ++r) CHECK(idx[r - 1] < idx[r], "%s: keep_idx not ascending at %lld", what, (long long)r);
  for (int64_t r = 0; r < nk; ++r)
    CHECK(idx[r] >= 0 && idx[r] < n && keep[idx[r]] == 1, "%s: keep_idx %lld not in the mask", what, (long long)r);
  CHECK(kept_min >= dropped_max, "%s: dropped %g above kept %g", what, dropped_max, kept_min);
}

static void rule_turn(int run, uint32_t* rule_bits_out) {
  const int L = 3, H_q = 8, H_kv = 2, D = 128, S = 24;
  const int64_t N = 40000, pi = 32, q_s = N - 64, q_e = N, C = 4096;
  const size_t nK = (size_t)L * H_kv * N * D, nQ = (size_t)L * H_q * S * D, nM = (size_t)L * H_q * D;
  rng_state = 0x1234567ull;
  float* hK = malloc(nK * 4);
  float* hQ = malloc(nQ * 4);
  for (size_t i = 0; i < nK; ++i) hK[i] = (float)uniform();
  float* dK = dalloc(nK * 4);
  float* dQ = dalloc(nQ * 4);
  float* dM = dalloc(nM * 4);
  up(dK, hK, nK * 4);
  hipStream_t st;
  HIP(hipStreamCreate(&st));
  for (int t = 0; t < 3; ++t) {
    for (size_t i = 0; i < nQ; ++i) hQ[i] = (float)uniform();
    up(dQ, hQ, nQ * 4);
    KVS(kvs_qmem_update(dQ, KVS_F32, L, H_q, S, D, 0.3f, t == 0, dM, st));
  }
  const size_t ws_b = kvs_rule_score_workspace(L, H_q, H_kv, N);
  void* ws = dalloc(ws_b);
  float* drule = dalloc(N * 4);
  KVS(kvs_rule_score(dK, KVS_F32, dM, L, H_q, H_kv, D, N, pi, q_s, q_e, drule, ws, ws_b, st));
  uint8_t* dkeep = dalloc(N);
  int32_t* didx = dalloc(N * 4);
  int64_t* dnk = dalloc(8);
  const size_t tws_b = kvs_topk_workspace(N);
  void* tws = dalloc(tws_b);
  KVS(kvs_topk_select(drule, N, 0, pi, q_s, q_e, C, dkeep, didx, dnk, tws, tws_b, st));
  int64_t* hslot = malloc(N * 8);
  for (int64_t j = 0; j < N; ++j) hslot[j] = 1000 + 3 * j;
  int64_t* dslot = dalloc(N * 8);
  int64_t* dslot2 = dalloc(N * 8);
  up(dslot, hslot, N * 8);
  KVS(kvs_slotmap_redirect(dslot, dkeep, N, -1, dslot2, st));
  /* the selection and the redirect in one launch, into other buffers */
  uint8_t* dkeep3 = dalloc(N);
  int32_t* didx3 = dalloc(N * 4);
  int64_t* dnk3 = dalloc(8);
  int64_t* dslot3 = dalloc(N * 8);
  KVS(kvs_topk_select_redirect(drule, N, 0, pi, q_s, q_e, C, dkeep3, didx3, dnk3, dslot, -1, dslot3, tws, tws_b, st));
  /* the no-allocation top-k on the same scores */
  uint8_t* dkeep2 = dalloc(N);
  int32_t* didx2 = dalloc(N * 4);
  int64_t* dnk2 = dalloc(8);
  KVS(kvs_topk_select_noalloc(drule, N, 0, pi, q_s, q_e, C, dkeep2, didx2, dnk2, st));
  HIP(hipStreamSynchronize(st));

  float* hM = malloc(nM * 4);
  float* hrule = malloc(N * 4);
  uint8_t *hkeep = malloc(N), *hkeep2 = malloc(N);
  int32_t *hidx = malloc(N * 4), *hidx2 = malloc(N * 4);
  int64_t hnk, hnk2, *hslot2 = malloc(N * 8);
  down(hM, dM, nM * 4);
  down(hrule, drule, N * 4);
  down(hkeep, dkeep, N);
  down(hidx, didx, N * 4);
  down(&hnk, dnk, 8);
  down(hslot2, dslot2, N * 8);
  down(hkeep2, dkeep2, N);
  down(hidx2, didx2, N * 4);
  down(&hnk2, dnk2, 8);
  for (int r = 0; r < L * H_q; ++r) {
    double s = 0;
    for (int d = 0; d < D; ++d) s += (double)hM[r * D + d] * hM[r * D + d];
    CHECK(fabs(sqrt(s) - 1.0) < 1e-5, "memory row %d norm %g", r, sqrt(s));
  }
  double total = 0;
  for (int64_t j = 0; j < N; ++j) {
    const int f = j < pi || (j >= q_s && j < q_e);
    if (f) CHECK(hrule[j] == 0.0f, "rule[%lld] on F is %g", (long long)j, hrule[j]);
    else CHECK(hrule[j] > 0.0f, "rule[%lld] = %g", (long long)j, hrule[j]);
    total += hrule[j];
  }
  CHECK(fabs(total - L * H_q) <= 1e-4 * L * H_q, "sum(rule) = %.8f, want %d", total, L * H_q);
  check_selection(hrule, N, 0, pi, q_s, q_e, C, hkeep, hidx, hnk, "rule top-k");
  CHECK(hnk2 == hnk && memcmp(hkeep2, hkeep, N) == 0 && memcmp(hidx2, hidx, hnk * 4) == 0,
        "no-allocation top-k differs from the workspace one");
  {
    uint8_t* k3 = malloc(N);
    int32_t* i3 = malloc(N * 4);
    int64_t n3, *s3 = malloc(N * 8);
    down(k3, dkeep3, N);
    down(i3, didx3, N * 4);
    down(&n3, dnk3, 8);
    down(s3, dslot3, N * 8);
    CHECK(n3 == hnk && memcmp(k3, hkeep, N) == 0 && memcmp(i3, hidx, hnk * 4) == 0 &&
              memcmp(s3, hslot2, N * 8) == 0,
          "top-k with the redirect fused differs from the two calls");
    free(k3);
    free(i3);
    free(s3);
  }
  for (int64_t j = 0; j < N; ++j)
    CHECK(hslot2[j] == (hkeep[j] ? hslot[j] : -1), "slot %lld: %lld", (long long)j, (long long)hslot2[j]);
  memcpy(rule_bits_out, hrule, N * 4);
  printf("rule turn %d: sum(rule) %.6f, n_kept %lld\n", run, total, (long long)hnk);

  free(hK); free(hQ); free(hM); free(hrule); free(hkeep); free(hkeep2); free(hidx); free(hidx2);
  free(hslot); free(hslot2);
  HIP(hipFree(dK)); HIP(hipFree(dQ)); HIP(hipFree(dM)); HIP(hipFree(ws)); HIP(hipFree(drule));
  HIP(hipFree(dkeep)); HIP(hipFree(didx)); HIP(hipFree(dnk)); HIP(hipFree(tws)); HIP(hipFree(dslot));
  HIP(hipFree(dslot2)); HIP(hipFree(dkeep2)); HIP(hipFree(didx2)); HIP(hipFree(dnk2));
  HIP(hipFree(dkeep3)); HIP(hipFree(didx3)); HIP(hipFree(dnk3)); HIP(hipFree(dslot3));
  HIP(hipStreamDestroy(st));
}

static void meank_step(void) {
  const int L = 2, H_q = 8, H_kv = 2, D = 128, blk = 32;
  const int64_t N = 32 * 400, nB = 400, Mq = 48, n_sink = 4, n_recent = 16, budget = 96, pool_pages = 128;
  const size_t nK = (size_t)L * H_kv * N * D, nQ = (size_t)L * H_q * Mq * D;
  rng_state = 0xabcdefull;
  uint16_t *hK = malloc(nK * 2), *hV = malloc(nK * 2), *hQ = malloc(nQ * 2);
  for (size_t i = 0; i < nK; ++i) hK[i] = to_bf16((float)uniform());
  for (size_t i = 0; i < nK; ++i) hV[i] = to_bf16((float)uniform());
  for (size_t i = 0; i < nQ; ++i) hQ[i] = to_bf16((float)(2.0 * uniform()));
  uint16_t *dK = dalloc(nK * 2), *dV = dalloc(nK * 2), *dQ = dalloc(nQ * 2);
  up(dK, hK, nK * 2);
  up(dV, hV, nK * 2);
  up(dQ, hQ, nQ * 2);
  const size_t nI = (size_t)L * H_kv * nB * D;
  uint16_t* dI = dalloc(nI * 2);
  KVS(kvs_meank_build(dK, L, H_kv, D, N, blk, 0, 0, 1e6, NULL, dI, NULL));
  const size_t ws_b = kvs_meank_score_workspace(L, H_q, H_kv, Mq, nB);
  void* ws = dalloc(ws_b);
  float* dR = dalloc(nB * 4);
  KVS(kvs_meank_score(dQ, dI, L, H_q, H_kv, D, Mq, nB, n_sink, n_recent, dR, ws, ws_b, NULL));
  uint8_t* dkeep = dalloc(nB);
  int32_t* didx = dalloc(nB * 4);
  int64_t* dnk = dalloc(8);
  KVS(kvs_topk_select(dR, nB, 0, n_sink, nB - n_recent, nB, budget, dkeep, didx, dnk, NULL, 0, NULL));
  int32_t* hpt = malloc(budget * 4);
  for (int64_t r = 0; r < budget; ++r) hpt[r] = (int32_t)((r * 37 + 11) % pool_pages);   /* distinct pages */
  int32_t* dpt = dalloc(budget * 4);
  up(dpt, hpt, budget * 4);
  const size_t nP = (size_t)L * H_kv * pool_pages * blk * D;
  uint16_t *dKp = dalloc(nP * 2), *dVp = dalloc(nP * 2);
  int32_t* derr = dalloc(4);
  HIP(hipMemset(derr, 0, 4));
  const int64_t pos_base = 5000;
  KVS(kvs_rerope_scatter(dK, dV, N, didx, dpt, budget, L, H_kv, D, blk, pos_base, 1e6, dKp, dVp, pool_pages, derr,
                         NULL));
  HIP(hipDeviceSynchronize());

  uint16_t* hI = malloc(nI * 2);
  float* hR = malloc(nB * 4);
  uint8_t* hkeep = malloc(nB);
  int32_t* hidx = malloc(nB * 4);
  int64_t hnk;
  int32_t herr;
  uint16_t *hKp = malloc(nP * 2), *hVp = malloc(nP * 2);
  down(hI, dI, nI * 2);
  down(hR, dR, nB * 4);
  down(hkeep, dkeep, nB);
  down(hidx, didx, nB * 4);
  down(&hnk, dnk, 8);
  down(&herr, derr, 4);
  down(hKp, dKp, nP * 2);
  down(hVp, dVp, nP * 2);
  /* index: every block of one (layer, head) against the float64 mean, within one bf16 ulp */
  for (int64_t b = 0; b < nB; ++b)
    for (int d = 0; d < D; ++d) {
      double m = 0;
      for (int t = 0; t < blk; ++t) m += from_bf16(hK[((size_t)1 * N + b * blk + t) * D + d]);
      m /= blk;
      const double got = from_bf16(hI[((size_t)1 * nB + b) * D + d]);
      const double ulp = ldexp(1.0, (int)floor(log2(fmax(fabs(m), 1e-30))) - 7);
      CHECK(fabs(got - m) <= ulp + 1e-5, "index block %lld dim %d: %g vs %g", (long long)b, d, got, m);
    }
  double total = 0;
  for (int64_t b = 0; b < nB; ++b) {
    const int f = b < n_sink || b >= nB - n_recent;
    if (f) CHECK(hR[b] == 0.0f, "R[%lld] forced is %g", (long long)b, hR[b]);
    total += hR[b];
  }
  CHECK(fabs(total - Mq) <= 1e-4 * Mq, "sum(R) = %.6f, want %lld", total, (long long)Mq);
  check_selection(hR, nB, 0, n_sink, nB - n_recent, nB, budget, hkeep, hidx, hnk, "Mean-K selection");
  CHECK(herr == 0, "scatter reported an out-of-range block");
  for (int lg = 0; lg < L * H_kv; ++lg)
    for (int64_t r = 0; r < budget; ++r)
      for (int t = 0; t < blk; ++t) {
        const size_t src = ((size_t)lg * N + (size_t)hidx[r] * blk + t) * D;
        const size_t dst = ((size_t)lg * pool_pages * blk + (size_t)hpt[r] * blk + t) * D;
        CHECK(memcmp(hVp + dst, hV + src, D * 2) == 0, "V page of block %lld differs", (long long)r);
        for (int i = 0; i < D / 2; ++i) {
          const double a = from_bf16(hK[src + i]), b2 = from_bf16(hK[src + i + D / 2]);
          const double c = from_bf16(hKp[dst + i]), e = from_bf16(hKp[dst + i + D / 2]);
          const double n0 = a * a + b2 * b2, n1 = c * c + e * e;
          CHECK(fabs(n0 - n1) <= n0 / 64 + 1e-6, "K pair norm changed: %g vs %g", n0, n1);
        }
      }
  printf("Mean-K step: sum(R) %.6f, n_kept %lld\n", total, (long long)hnk);
  free(hK); free(hV); free(hQ); free(hI); free(hR); free(hkeep); free(hidx); free(hpt); free(hKp); free(hVp);
  HIP(hipFree(dK)); HIP(hipFree(dV)); HIP(hipFree(dQ)); HIP(hipFree(dI)); HIP(hipFree(ws)); HIP(hipFree(dR));
  HIP(hipFree(dkeep)); HIP(hipFree(didx)); HIP(hipFree(dnk)); HIP(hipFree(dpt)); HIP(hipFree(dKp));
  HIP(hipFree(dVp)); HIP(hipFree(derr));
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    fprintf(stderr, "no GPU\n");
    return 102;
  }
  const int64_t N = 40000;
  uint32_t* a = malloc(N * 4);
  uint32_t* b = malloc(N * 4);
  rule_turn(0, a);
  rule_turn(1, b);
  CHECK(memcmp(a, b, N * 4) == 0, "rule scores differ between two identical runs");
  meank_step();
  free(a);
  free(b);
  printf("kvs_c_consumer: %d failed checks\n", failures);
  return failures;
}
