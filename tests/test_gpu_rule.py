"""GPU parity, IntentKV rule mode: QueryMemory, rule score, top-k, slot redirect.

Every case feeds the same seeded tensors to the HIP library (through the C ABI)
and to the float64 oracle.  Tolerances: QueryMemory 1e-5 absolute; rule scores
2e-3 relative per candidate (float32 accumulation against float64); top-k and
slot maps bit-exact when both sides rank the same float32 scores -- at full size
the oracle's selection runs on the GPU's own scores, stage by stage, after those
scores have been checked against the oracle's; and the selection made on the
GPU's scores must also be a valid top-C* under the oracle's own scores up to
that score tolerance.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_space_retrieval_amd import kvs, workloads as W
from tests.helpers import assert_rel, assert_valid_selection, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RULE_RTOL = 2e-3


def gpu_rule(K, M, pi, q_s, q_e):
    r = kvs.kvs_rule_score(K, M, pi, q_s, q_e)
    torch.cuda.synchronize()
    return r


def check_rule(K, M, pi, q_s, q_e, what, M_oracle=None):
    """M_oracle: the oracle's own QueryMemory when M came from the GPU."""
    got = gpu_rule(K, M, pi, q_s, q_e).cpu().numpy()
    want = oracle.rule_score(host(K), host(M) if M_oracle is None else M_oracle, pi, q_s, q_e)
    F = oracle.forced_mask(K.shape[2], pi, q_s, q_e)
    assert np.all(got[F] == 0.0), f"{what}: forced positions must score exactly 0"
    if (~F).any():
        assert_rel(got[~F], want[~F], RULE_RTOL, what)
        L, H_q = M.shape[0], M.shape[1]
        assert abs(got.sum(dtype=np.float64) - L * H_q) <= 1e-4 * L * H_q
    return got, want


# ---------------------------------------------------------------- QueryMemory

@pytest.mark.parametrize("dtype,D,S", [("f32", 64, 32), ("bf16", 128, 64), ("bf16", 64, 5),
                                       # spans over several load batches with a ragged last one
                                       ("f32", 128, 70), ("bf16", 128, 200), ("f32", 64, 97), ("bf16", 64, 300)])
def test_qmem_turns(dtype, D, S):
    L, H_q, T, lam = 3, 8, 4, 0.3
    spans = [W.normal((L, H_q, S, D), 77, 100 + t, dtype, DEV) for t in range(T)]
    M = torch.empty((L, H_q, D), dtype=torch.float32, device=DEV)
    Mo = None
    for t, q in enumerate(spans):
        kvs.kvs_qmem_update(q, lam, M, first_turn=(t == 0))
        Mo = oracle.qmem_update(host(q), lam, Mo)
        torch.cuda.synchronize()
        np.testing.assert_allclose(M.cpu().numpy(), Mo, rtol=0, atol=1e-5)


def test_qmem_query_mode_and_zero():
    L, H_q, S, D = 2, 4, 8, 128
    q0 = W.normal((L, H_q, S, D), 78, 1, "bf16", DEV)
    q1 = W.normal((L, H_q, S, D), 78, 2, "bf16", DEV)
    M = torch.full((L, H_q, D), float("nan"), device=DEV)     # first turn must not read M
    kvs.kvs_qmem_update(q0, math.inf, M, True)
    kvs.kvs_qmem_update(q1, math.inf, M, False)
    torch.cuda.synchronize()
    np.testing.assert_allclose(M.cpu().numpy(), oracle.qmem_update(host(q1), math.inf), atol=1e-5)
    z = torch.zeros((1, 2, 3, 64), device=DEV)
    Mz = torch.empty((1, 2, 64), device=DEV)
    kvs.kvs_qmem_update(z, 0.5, Mz, True)
    torch.cuda.synchronize()
    assert torch.all(Mz == 0)


def test_qmem_checkpoint_and_resume_is_bit_exact():
    """M_t is the whole per-session state of the rule mode (IntentKV Sec. 3.2): t turns, a round trip
    of M through host memory (a session saved and restored), then the remaining turns equal all
    turns run at once, bit for bit -- M and the rule scores that read it."""
    L, H_q, H_kv, S, D, N, T, lam = 3, 8, 2, 40, 128, 3000, 6, 0.3
    spans = [W.normal((L, H_q, S, D), 79, 200 + t, "bf16", DEV) for t in range(T)]
    K = W.normal((L, H_kv, N, D), 79, W.T_K, "bf16", DEV)
    M_all = torch.empty((L, H_q, D), dtype=torch.float32, device=DEV)
    for t, q in enumerate(spans):
        kvs.kvs_qmem_update(q, lam, M_all, t == 0)
    for cut in (1, 3, 5):
        M = torch.empty((L, H_q, D), dtype=torch.float32, device=DEV)
        for t in range(cut):
            kvs.kvs_qmem_update(spans[t], lam, M, t == 0)
        torch.cuda.synchronize()
        saved = M.cpu().numpy().copy()                      # checkpoint
        del M
        M = torch.from_numpy(saved).to(DEV)                 # resume in a fresh buffer
        for t in range(cut, T):
            kvs.kvs_qmem_update(spans[t], lam, M, False)
        torch.cuda.synchronize()
        assert torch.equal(M.view(torch.int32), M_all.view(torch.int32)), f"resume after {cut} turns"
        a = kvs.kvs_rule_score(K, M, 5, N - 64, N).clone()
        b = kvs.kvs_rule_score(K, M_all, 5, N - 64, N)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ---------------------------------------------------------------- rule score

def test_rule_tiny_config():
    c = W.config("rule-tiny")
    inp = W.rule_inputs(c, DEV)
    M = torch.empty((c["L"], c["H_q"], c["D"]), dtype=torch.float32, device=DEV)
    Mo = None
    for t, q in enumerate(inp["spans"]):
        kvs.kvs_qmem_update(q, c["lam"], M, t == 0)
        Mo = oracle.qmem_update(host(q), c["lam"], Mo)
    check_rule(inp["K"], M, c["pi"], c["q_s"], c["q_e"], "rule-tiny", M_oracle=Mo)


@pytest.mark.parametrize("L,H_q,H_kv,D,N,pi,q_s,q_e", [
    (2, 32, 8, 128, 5000, 64, 4900, 4964),     # 3 chunks, ragged tail, G = 4
    (3, 40, 8, 128, 4097, 1, 4097, 4097),      # G = 5, one-row tail chunk, empty span
    (2, 8, 8, 128, 300, 0, 0, 0),              # G = 1, no forced positions
    (1, 24, 2, 128, 2100, 10, 20, 30),         # G = 12: two 8-head groups
    (2, 16, 4, 64, 3000, 5, 2990, 3000),       # D = 64
    (1, 4, 2, 128, 1, 0, 0, 0),                # N = 1
    (1, 16, 2, 128, 777, 3, 700, 720),         # G = 8: both spill halves of one 8-head group
    (1, 32, 2, 64, 90, 0, 80, 90),             # G = 16, D = 64, fewer rows than one tile pair per wave
])
def test_rule_bf16_shapes(L, H_q, H_kv, D, N, pi, q_s, q_e):
    K = W.normal((L, H_kv, N, D), 11, W.T_K, "bf16", DEV)
    M = W.memory_vectors(L, H_q, D, 11, DEV)
    check_rule(K, M, pi, q_s, q_e, f"rule L{L} Hq{H_q} Hkv{H_kv} D{D} N{N}")


@pytest.mark.parametrize("dtype,L,H_q,H_kv,D,N", [
    ("bf16", 1, 8, 2, 128, 131073),    # 65 chunks of 2048, one-row tail
    ("f32", 1, 4, 2, 64, 131073),      # float32 keys, long cache
    ("f32", 2, 24, 2, 128, 1500),      # float32 keys, G = 12
    ("bf16", 2, 32, 8, 128, 2049),     # two chunks, the second one row long
])
def test_rule_long_and_f32(dtype, L, H_q, H_kv, D, N):
    K = W.normal((L, H_kv, N, D), 14, W.T_K, dtype, DEV)
    M = W.memory_vectors(L, H_q, D, 14, DEV)
    check_rule(K, M, 7, N - 100, N - 40, f"rule {dtype} L{L} Hq{H_q} Hkv{H_kv} D{D} N{N}")


def test_rule_large_logits_keep_precision():
    # |M| ~ 10 and K spread ~ 3: logits of tens; the hi/lo split of M keeps them exact enough.
    L, H_q, H_kv, D, N = 1, 8, 2, 128, 3000
    K = W.normal((L, H_kv, N, D), 12, W.T_K, "bf16", DEV, scale=3.0)
    M = W.memory_vectors(L, H_q, D, 12, DEV) * 1.0
    check_rule(K, M, 0, 0, 0, "large logits")


@pytest.mark.parametrize("scale,G", [(60.0, 4), (100.0, 4), (100.0, 5)])
def test_rule_wide_logit_range_escapes(scale, G):
    # Logits spread over hundreds of log2 units: chunk maxima differ by far more
    # than float32's exponent range of exp2 terms, so the per-chunk (max, sum)
    # merge must rescale without overflow or flushing the chunks that matter,
    # and every candidate, down to the tiny ones, must still meet the tolerance.
    L, H_kv, D, N = 2, 2, 128, 2500
    K = W.normal((L, H_kv, N, D), 15, W.T_K, "bf16", DEV, scale=scale)
    M = W.memory_vectors(L, H_kv * G, D, 15, DEV)
    check_rule(K, M, 3, 2400, 2450, f"wide logits scale {scale} G {G}")


def test_rule_all_forced_and_determinism():
    L, H_q, H_kv, D, N = 2, 8, 2, 128, 700
    K = W.normal((L, H_kv, N, D), 13, W.T_K, "bf16", DEV)
    M = W.memory_vectors(L, H_q, D, 13, DEV)
    assert torch.all(gpu_rule(K, M, 400, 300, 700) == 0)
    a = gpu_rule(K, M, 3, 600, 650).clone()
    b = gpu_rule(K, M, 3, 600, 650)
    assert torch.equal(a, b)


def _spilled_fraction(ws, L, H_q, N):
    """The workspace starts with the [L*H_q, N] float32 spill; filled with 0xff before a call, the
    share of it written afterwards is the share of positions whose chunk took the spill path."""
    spill = ws[: L * H_q * N * 4].view(torch.int32)
    return float((spill != -1).sum().item()) / (L * H_q * N)


@pytest.mark.parametrize("L,H_q,H_kv,D,N,paged", [
    (2, 32, 8, 128, 5000, False),    # G = 4, ragged tail
    (3, 40, 8, 128, 4097, False),    # G = 5, one-row tail chunk
    (1, 16, 2, 128, 777, True),      # G = 8, read through a slot map
    (2, 16, 4, 64, 3000, True),      # D = 64
    (1, 8, 2, 128, 131073, False),   # many chunks per group
])
def test_rule_fold_equals_spill_path(L, H_q, H_kv, D, N, paged):
    """The bf16 scorer folds each chunk's G heads on chip once its group's normalisers are out, and
    spills the chunk when they are not; the column pass finishes a spilled chunk with the fold's
    own arithmetic.  Every chunk spilled (wait limit < 0), no waiting at all (limit 0) and the
    default all give the same bits, and the default folds (nothing written to the spill)."""
    if paged:
        _, pool, slots, M = _paged_inputs(L, H_q, H_kv, D, N, N + 500, "bf16", 21, dead=(3,))
        run = lambda ws: kvs.kvs_rule_score_paged(pool, slots, M, 5, N - 70, N - 10, ws=ws)
    else:
        K = W.normal((L, H_kv, N, D), 21, W.T_K, "bf16", DEV)
        M = W.memory_vectors(L, H_q, D, 21, DEV)
        run = lambda ws: kvs.kvs_rule_score(K, M, 5, N - 70, N - 10, ws=ws)
    need = kvs.kvs_rule_score_workspace(L, H_q, H_kv, N)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = {}
    prev = kvs.kvs_rule_score_wait_limit(-1)
    try:
        for limit in (-1, 0, prev):
            kvs.kvs_rule_score_wait_limit(limit)
            ws.fill_(0xFF)
            out[limit] = run(ws).clone()
            torch.cuda.synchronize()
            if limit == -1:
                assert _spilled_fraction(ws, L, H_q, N) == 1.0
            if limit == prev and N <= 5000:
                assert _spilled_fraction(ws, L, H_q, N) == 0.0
    finally:
        kvs.kvs_rule_score_wait_limit(prev)
    for limit in (0, prev):
        assert torch.equal(out[limit].view(torch.int32), out[-1].view(torch.int32)), f"limit {limit}"
    if not paged:
        F = oracle.forced_mask(N, 5, N - 70, N - 10)
        want = oracle.rule_score(host(K), host(M), 5, N - 70, N - 10)
        assert_rel(out[prev].cpu().numpy()[~F], want[~F], RULE_RTOL, "fold path")


@pytest.mark.parametrize("name", ["rule-8b", "rule-14b"])
def test_rule_full_size(name):
    """Full configuration in the benchmark's launch shape, every output against the oracle."""
    c = W.config(name)
    print(f"[{name}] generating inputs", flush=True)
    inp = W.rule_inputs(c, DEV)
    M = torch.empty((c["L"], c["H_q"], c["D"]), dtype=torch.float32, device=DEV)
    Mo = None
    for t, q in enumerate(inp["spans"]):
        kvs.kvs_qmem_update(q, c["lam"], M, t == 0)
        Mo = oracle.qmem_update(host(q), c["lam"], Mo)
    torch.cuda.synchronize()
    np.testing.assert_allclose(M.cpu().numpy(), Mo, atol=1e-5)
    print(f"[{name}] oracle rule score", flush=True)
    got, want = check_rule(inp["K"], M, c["pi"], c["q_s"], c["q_e"], name, M_oracle=Mo)
    ws = torch.full((kvs.kvs_rule_score_workspace(c["L"], c["H_q"], c["H_kv"], c["N"]),), 0xFF,
                    dtype=torch.uint8, device=DEV)
    again = kvs.kvs_rule_score(inp["K"], M, c["pi"], c["q_s"], c["q_e"], ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy().view(np.int32), got.view(np.int32))
    spilled = _spilled_fraction(ws, c["L"], c["H_q"], c["N"])
    print(f"[{name}] share of positions spilled: {spilled:.4f}", flush=True)
    assert spilled < 0.05
    # top-k and slot redirect in the benchmark's launch shape (workspace: the multi-workgroup path
    # above 32768 scores), bit for bit against the oracle's selection of the same float32 scores
    keep, idx, nk = kvs.kvs_topk_select(torch.from_numpy(got).to(DEV), (0, c["pi"]),
                                        (c["q_s"], c["q_e"]), c["C"])
    slots = kvs.kvs_slotmap_redirect(inp["slots"], keep, c["dead_slot"])
    torch.cuda.synchronize()
    nk = int(nk.item())
    o_keep, o_idx, o_nk = oracle.topk_select(got, (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"])
    assert nk == o_nk == c["C"]
    np.testing.assert_array_equal(keep.cpu().numpy(), o_keep.astype(np.uint8))
    np.testing.assert_array_equal(idx[:nk].cpu().numpy(), o_idx)
    np.testing.assert_array_equal(slots.cpu().numpy(), oracle.slotmap_redirect(host(inp["slots"]), o_keep,
                                                                               c["dead_slot"]))
    # and it is a valid top-C* under the oracle's own scores, up to the score tolerance
    F = oracle.forced_mask(c["N"], c["pi"], c["q_s"], c["q_e"])
    assert_valid_selection(want, o_idx, F, c["C"] - int(F.sum()), 2 * RULE_RTOL)


# ---------------------------------------------------------------- rule score through the slot map

def _paged_inputs(L, H_q, H_kv, D, N, pool_size, dtype, seed, dead=()):
    """Token-major pool with the cache's rows at a seeded permutation of slots (some dead)."""
    K = W.normal((L, H_kv, N, D), seed, W.T_K, dtype, DEV)
    pool = W.normal((L, pool_size, H_kv, D), seed, W.T_K + 30, dtype, DEV)
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(pool_size)[:N].copy()).to(DEV)
    pool[:, perm] = K.permute(0, 2, 1, 3)
    slots = perm.clone()
    if len(dead):
        slots[list(dead)] = -1
    M = W.memory_vectors(L, H_q, D, seed, DEV)
    return K, pool, slots, M


@pytest.mark.parametrize("dtype,L,H_q,H_kv,D,N,pool_size,dead", [
    ("bf16", 2, 32, 8, 128, 5000, 6000, (7, 8, 4000)),
    ("bf16", 1, 24, 2, 64, 2100, 2100, ()),
    ("f32", 2, 4, 2, 64, 1024, 1500, (0, 1023)),
])
def test_rule_paged_against_oracle(dtype, L, H_q, H_kv, D, N, pool_size, dead):
    K, pool, slots, M = _paged_inputs(L, H_q, H_kv, D, N, pool_size, dtype, 15, dead)
    pi, q_s, q_e = 16, N - 64, N
    got = kvs.kvs_rule_score_paged(pool, slots, M, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.rule_score_paged(host(pool), slots.cpu().numpy(), host(M), pi, q_s, q_e)
    out = oracle.forced_mask(N, pi, q_s, q_e)
    out[list(dead)] = True
    assert np.all(got[out] == 0.0)
    assert_rel(got[~out], want[~out], RULE_RTOL, f"paged rule {dtype} D{D}")


@pytest.mark.parametrize("name", ["rule-8b", "rule-14b"])
def test_rule_paged_full_size_equals_dense(name):
    """At full size, the pool read through a permuted slot map gives the dense scores.  The two
    calls score the same keys in chunks of different lengths (the paged chunk is shorter, to keep
    three workgroups per CU beside its slot array), so the softmax partials merge in a different
    grouping: the scores agree to float32 summation order, 1e-5 relative -- a wrong row would be
    off by orders of magnitude -- and the forced positions are exactly 0 in both."""
    c = W.config(name)
    L, H_q, H_kv, D, N = c["L"], c["H_q"], c["H_kv"], c["D"], c["N"]
    K, pool, slots, M = _paged_inputs(L, H_q, H_kv, D, N, N + 4096, "bf16", 16)
    dense = kvs.kvs_rule_score(K, M, c["pi"], c["q_s"], c["q_e"])
    paged = kvs.kvs_rule_score_paged(pool, slots, M, c["pi"], c["q_s"], c["q_e"])
    torch.cuda.synchronize()
    d, p = dense.cpu().numpy().astype(np.float64), paged.cpu().numpy().astype(np.float64)
    F = oracle.forced_mask(N, c["pi"], c["q_s"], c["q_e"])
    assert np.all(d[F] == 0) and np.all(p[F] == 0)
    rel = np.abs(p[~F] - d[~F]) / d[~F]
    print(f"[{name}] paged vs dense: max relative difference {rel.max():.2e}", flush=True)
    assert rel.max() <= 1e-5
    del K, pool


# ---------------------------------------------------------------- window score

@pytest.mark.parametrize("L,H_q,H_kv,N,Wn,pi,q_s,q_e", [
    (2, 32, 8, 5000, 32, 64, 4936, 5000),      # span at the end: candidates [pi, q_s)
    (2, 8, 2, 3000, 16, 10, 1000, 1100),       # span in the middle: a hole in the candidates
    (1, 40, 8, 777, 7, 0, 0, 0),               # G = 5, odd W, no forced positions, ragged N
    (1, 4, 4, 300, 1, 299, 0, 0),              # one candidate
    (1, 16, 2, 2500, 32, 5, 2400, 2450),       # G*W = 256 rows: pass 1 with four-wave workgroups
    (1, 20, 4, 1800, 40, 0, 1700, 1800),       # G*W = 200 rows (padded to 224): four waves, a partial one
    (1, 40, 4, 1500, 32, 3, 1400, 1450),       # G*W = 320 rows: pass 1 with a second, partial 256-row tile
])
@pytest.mark.parametrize("D", [128, 64])
def test_window_score_against_oracle(L, H_q, H_kv, N, Wn, pi, q_s, q_e, D):
    """Wn window rows per query head, head dimension D."""
    K = W.normal((L, H_kv, N, D), 17, W.T_K, "bf16", DEV)
    Qw = W.normal((L, H_q, Wn, D), 17, W.T_Q, "bf16", DEV)
    got = kvs.kvs_window_score(K, Qw, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.window_score(host(K), host(Qw), pi, q_s, q_e)
    F = oracle.forced_mask(N, pi, q_s, q_e)
    assert np.all(got[F] == 0.0)
    assert_rel(got[~F], want[~F], RULE_RTOL, f"window score W{Wn} N{N} D{D}")
    assert abs(got.sum(dtype=np.float64) - L * H_q * Wn) <= 1e-4 * L * H_q * Wn


def test_window_one_row_matches_rule_score():
    """W = 1 with the QueryMemory as the window row gives the rule score (to float32 rounding)."""
    L, H_q, H_kv, N, D = 2, 16, 4, 4000, 128
    K = W.normal((L, H_kv, N, D), 18, W.T_K, "bf16", DEV)
    M = W.memory_vectors(L, H_q, D, 18, DEV)
    Mb = M.to(torch.bfloat16)
    rule = kvs.kvs_rule_score(K, Mb.float(), 5, 3990, 4000)
    win = kvs.kvs_window_score(K, Mb[:, :, None, :].contiguous(), 5, 3990, 4000)
    torch.cuda.synchronize()
    F = oracle.forced_mask(N, 5, 3990, 4000)
    assert_rel(win.cpu().numpy()[~F], rule.cpu().numpy()[~F], RULE_RTOL, "window(W=1) vs rule")


@pytest.mark.parametrize("name", ["rule-8b", "rule-14b"])
def test_window_score_full_size_sampled(name):
    """The cache with a 32-row window (128 rows per KV group at rule-8b, 160 at rule-14b): two
    layers' contribution checked against the oracle, the whole call by its invariants."""
    c = W.config(name)
    L, H_q, H_kv, D, N = c["L"], c["H_q"], c["H_kv"], c["D"], c["N"]
    K = W.normal((L, H_kv, N, D), c["seed"], W.T_K, "bf16", DEV)
    Qw = W.normal((L, H_q, 32, D), c["seed"], W.T_Q, "bf16", DEV)
    got = kvs.kvs_window_score(K, Qw, c["pi"], c["q_s"], c["q_e"])
    # two layers alone, through the same library call, against the oracle
    two = kvs.kvs_window_score(K[:2].contiguous(), Qw[:2].contiguous(), c["pi"], c["q_s"], c["q_e"])
    torch.cuda.synchronize()
    F = oracle.forced_mask(N, c["pi"], c["q_s"], c["q_e"])
    want = oracle.window_score(host(K[:2]), host(Qw[:2]), c["pi"], c["q_s"], c["q_e"])
    assert_rel(two.cpu().numpy()[~F], want[~F], RULE_RTOL, f"window score, 2 layers of {name}")
    g = got.cpu().numpy()
    assert np.all(g[F] == 0.0) and np.all(g[~F] > 0.0)
    assert abs(g.sum(dtype=np.float64) - L * H_q * 32) <= 1e-4 * L * H_q * 32
    del K, Qw


# ---------------------------------------------------------------- top-k

def check_topk(score, f0, f1, C, single_workgroup=False):
    keep, idx, nk = kvs.kvs_topk_select(score, f0, f1, C, single_workgroup=single_workgroup)
    torch.cuda.synchronize()
    ok, oidx, onk = oracle.topk_select(score.cpu().numpy(), f0, f1, C)
    nk = int(nk.item())
    assert nk == onk
    np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), ok)
    np.testing.assert_array_equal(idx[:nk].cpu().numpy(), oidx)


@pytest.mark.parametrize("n,single", [(5, False), (77, False), (1025, False), (4097, False), (4098, False),
                                      (4099, False), (8191, False), (8193, False), (32767, False),
                                      (32769, False), (92161, False), (40001, True)])
@pytest.mark.parametrize("offset", [0, 1])
def test_topk_ragged_tail_candidates(n, single, offset):
    """No forced range, and the largest scores at the last three positions: a selection whose last
    16-byte load of scores is only partly inside n must still see them.  offset = 1 views the
    scores, the mask and the indices one element into their allocations (4, 1 and 4 bytes past
    a 16-byte boundary)."""
    base = W.scores_with_ties(n + offset, 900 + n, None).clone()
    for i, v in enumerate((100.0, 99.0, 98.0)):
        if n - 1 - i >= 0:
            base[offset + n - 1 - i] = v
    score = base.to(DEV)[offset:]
    for C in (1, 3, n // 2 + 1):
        print(f"[topk tail] n={n} offset={offset} single={single} C={C}", flush=True)
        keep = torch.full((n + offset,), 7, dtype=torch.uint8, device=DEV)[offset:]
        idx = torch.full((n + offset,), -5, dtype=torch.int32, device=DEV)[offset:]
        keep, idx, nk = kvs.kvs_topk_select(score, (0, 0), (0, 0), C, keep_mask=keep, keep_idx=idx,
                                            single_workgroup=single)
        torch.cuda.synchronize()
        ok, oidx, onk = oracle.topk_select(score.cpu().numpy(), (0, 0), (0, 0), C)
        nk = int(nk.item())
        assert nk == onk == min(C, n)
        np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), ok)
        np.testing.assert_array_equal(idx[:nk].cpu().numpy(), oidx)
        assert set(range(max(0, n - min(C, 3)), n)) <= set(oidx.tolist())


@pytest.mark.parametrize("n,levels,f0,f1,C", [
    (1024, None, (0, 16), (992, 1024), 256),
    (1024, 7, (0, 16), (992, 1024), 256),          # heavy ties at the threshold
    (32768, 50, (0, 64), (32704, 32768), 8192),
    (92160, None, (0, 64), (92096, 92160), 8192),
    (92160, 3, (0, 64), (92096, 92160), 8192),
    (8192, 1000, (0, 4), (8128, 8192), 2048),      # Mean-K shape
    (4097, 2, (5, 3000), (2000, 4097), 3500),      # overlapping forced ranges
    (1, None, (0, 0), (0, 0), 1),
    (77, None, (0, 0), (0, 0), 0),                 # C = 0
    (500, None, (0, 10), (490, 500), 5),           # C < |F|
    (500, None, (0, 10), (490, 500), 10000),       # C >= n
    (0, None, (0, 0), (0, 0), 5),                  # empty input
    (8192, None, (0, 0), (0, 0), 1),               # register kernel size limits and one past them
    (8193, 4, (0, 1), (8192, 8193), 4000),
    (32768, None, (0, 64), (32704, 32768), 8192),
    (32769, None, (0, 64), (32705, 32769), 8192),
    (1025, None, (1000, 1025), (0, 0), 1),
])
def test_topk_bit_exact(n, levels, f0, f1, C):
    score = W.scores_with_ties(n, n + 1, levels).to(DEV)
    check_topk(score, f0, f1, C)
    if n > 32768:   # the no-workspace single-workgroup path as well
        check_topk(score, f0, f1, C, single_workgroup=True)


@pytest.mark.parametrize("n,levels,C,f0,f1", [
    (65537, None, 1, (0, 0), (0, 0)),                 # one kept, ragged last slice
    (200000, 9, 150000, (10, 100000), (99990, 100010)),  # heavy ties, overlapping forced ranges
    (100000, None, 30, (0, 64), (99936, 100000)),     # C < |F| -> forced only
    (70000, 1, 40000, (0, 5), (69990, 70000)),        # every candidate ties
])
def test_topk_multi_workgroup(n, levels, C, f0, f1):
    score = W.scores_with_ties(n, n + 7, levels).to(DEV)
    check_topk(score, f0, f1, C)
    check_topk(score, f0, f1, C, single_workgroup=True)


def test_topk_multi_workgroup_repeatable():
    """Slices add their histograms with atomics in whatever order they arrive:
    the selection must not depend on it (integer sums), call after call."""
    n = 150000
    score = W.scores_with_ties(n, 31, 40).to(DEV)
    first = [t.clone() for t in kvs.kvs_topk_select(score, (0, 10), (n - 10, n), 20000)]
    for _ in range(5):
        again = kvs.kvs_topk_select(score, (0, 10), (n - 10, n), 20000)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a[: int(first[2].item())] if a.dtype == torch.int32 else a,
                               b[: int(first[2].item())] if b.dtype == torch.int32 else b)


@pytest.mark.parametrize("n,C", [(32768, 8192), (92160, 8192), (8192, 2048)])
def test_topk_concentrated_scores(n, C):
    """Rule-score-like keys: every value within a few 1e-3 of the mean, so the
    candidates share their high key bits and the radix passes run on the low ones."""
    x = W.scores_with_ties(n, 4242)
    score = (0.0353 * (1.0 + 0.0026 * x)).float().to(DEV)
    check_topk(score, (0, 64), (n - 64, n), C)
    if n > 32768:
        check_topk(score, (0, 64), (n - 64, n), C, single_workgroup=True)


@pytest.mark.parametrize("n,C,spread", [(32768, 8192, 1e-6), (8192, 3000, 1e-5), (32768, 20000, 0.0),
                                         (92160, 8192, 1e-6)])
def test_topk_cluster_with_outliers(n, C, spread):
    """A dense cluster and a few far outliers: the first 11-bit digit of the candidates' key range
    puts the whole cluster into one bin, far more keys than the one-workgroup kernel ranks directly,
    so its 8-bit passes over the keys in registers find the threshold (spread 0: every cluster key
    ties)."""
    g = np.random.default_rng([n, 17])
    x = 1.0 + spread * g.standard_normal(n)
    x[g.choice(n, 16, replace=False)] = 1e3 * (1.0 + g.random(16))
    score = torch.from_numpy(x.astype(np.float32)).to(DEV)
    check_topk(score, (0, 4), (n - 64, n), C)


def test_topk_special_values():
    s = torch.tensor([float("nan"), -float("inf"), 0.0, -0.0, 1.0, float("inf"), -1e-30, 1e-30,
                      float("nan"), 0.0], device=DEV)
    for C in range(0, 11):
        check_topk(s, (0, 0), (0, 0), C)
    check_topk(s, (4, 6), (0, 1), 5)


def test_topk_all_equal():
    s = torch.full((10000,), 0.25, device=DEV)
    check_topk(s, (0, 3), (9990, 10000), 1000)


# ---------------------------------------------------------------- slot map

def test_slotmap_bit_exact():
    c = W.config("rule-tiny")
    score = W.scores_with_ties(c["N"], 5).to(DEV)
    keep, idx, nk = kvs.kvs_topk_select(score, (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"])
    slots = W.rule_inputs(c, DEV)["slots"]
    out = kvs.kvs_slotmap_redirect(slots, keep, c["dead_slot"])
    torch.cuda.synchronize()
    want = oracle.slotmap_redirect(slots.cpu().numpy(), keep.cpu().numpy().astype(bool), c["dead_slot"])
    np.testing.assert_array_equal(out.cpu().numpy(), want)
    assert int((out == -1).sum()) == c["N"] - c["C"]
    kvs.kvs_slotmap_redirect(slots, keep, 123456789, slot_out=slots)      # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(slots.cpu().numpy(), np.where(want == -1, 123456789, want))


@pytest.mark.parametrize("n,C,f0,f1,single,in_place", [
    (5000, 700, (0, 16), (4900, 4964), False, False),        # one workgroup, keys in registers (8 per thread, two 16-byte loads)
    (30000, 4096, (0, 64), (29936, 30000), False, True),     # 32 per thread, slots redirected in place
    (92160, 8192, (0, 64), (92096, 92160), False, False),    # several workgroups
    (92160, 8192, (0, 64), (92096, 92160), True, True),      # one workgroup streaming from L2
    (3000, 5000, (0, 10), (2990, 3000), False, False),       # C >= n: everything kept
    (3000, 20, (0, 10), (2980, 3000), False, False),         # C < |F|: the forced set only
    (1, 1, (0, 0), (0, 0), False, False),
])
def test_topk_select_redirect_equals_the_two_calls(n, C, f0, f1, single, in_place):
    """The fused selection + redirect writes the same mask, indices, count and slot map, bit for bit,
    as kvs_topk_select followed by kvs_slotmap_redirect, on every top-k path."""
    score = W.scores_with_ties(n, n + 3, 64).to(DEV)                      # many ties at the threshold
    slots = torch.from_numpy(np.random.default_rng(n).permutation(4 * n)[:n].copy()).to(DEV)
    keep, idx, nk = kvs.kvs_topk_select(score, f0, f1, C, single_workgroup=single)
    want_slots = kvs.kvs_slotmap_redirect(slots, keep, -7)
    s_in = slots.clone()
    k2, i2, n2, s_out = kvs.kvs_topk_select_redirect(score, f0, f1, C, s_in, -7,
                                                     slot_out=s_in if in_place else None, single_workgroup=single)
    torch.cuda.synchronize()
    m = int(nk.item())
    assert int(n2.item()) == m
    assert torch.equal(keep, k2) and torch.equal(idx[:m], i2[:m])
    assert torch.equal(s_out, want_slots)
    if in_place:
        assert s_out.data_ptr() == s_in.data_ptr()


def test_rule_turn_end_to_end_tiny():
    """qmem x 3 turns -> rule -> top-k -> slot map on rule-tiny, against the oracle chain."""
    c = W.config("rule-tiny")
    inp = W.rule_inputs(c, DEV)
    M = torch.empty((c["L"], c["H_q"], c["D"]), dtype=torch.float32, device=DEV)
    Mo = None
    for t, q in enumerate(inp["spans"]):
        kvs.kvs_qmem_update(q, c["lam"], M, t == 0)
        Mo = oracle.qmem_update(host(q), c["lam"], Mo)
    rule = kvs.kvs_rule_score(inp["K"], M, c["pi"], c["q_s"], c["q_e"])
    keep, idx, nk = kvs.kvs_topk_select(rule, (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"])
    slots = kvs.kvs_slotmap_redirect(inp["slots"], keep, c["dead_slot"])
    torch.cuda.synchronize()
    o_rule = oracle.rule_score(host(inp["K"]), Mo, c["pi"], c["q_s"], c["q_e"])
    F = oracle.forced_mask(c["N"], c["pi"], c["q_s"], c["q_e"])
    assert_rel(rule.cpu().numpy()[~F], o_rule[~F], RULE_RTOL, "chain rule")
    nk = int(nk.item())
    assert nk == c["C"]
    kidx = idx[:nk].cpu().numpy()
    assert_valid_selection(o_rule, kidx, F, c["C"] - int(F.sum()), 2 * RULE_RTOL)
    s = slots.cpu().numpy()
    kept = np.zeros(c["N"], bool); kept[kidx] = True
    np.testing.assert_array_equal(s[kept], inp["slots"].cpu().numpy()[kept])
    assert np.all(s[~kept] == c["dead_slot"])
    # stage by stage: the oracle's selection and slot map on the GPU's scores, bit for bit
    o_keep, o_idx, _ = oracle.topk_select(rule.cpu().numpy(), (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"])
    np.testing.assert_array_equal(kidx, o_idx)
    np.testing.assert_array_equal(s, oracle.slotmap_redirect(host(inp["slots"]), o_keep, c["dead_slot"]))
