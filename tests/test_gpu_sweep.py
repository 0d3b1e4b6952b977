"""GPU parity over seeded random shapes: each case draws its sizes, forced
ranges and budgets from its seed (printed before it runs) and checks the whole
chain against the float64 oracle at the same bars as the targeted tests --
rule and window scores and R_b within 2e-3 relative per candidate, the index
and re-RoPE'd K within 1 ulp, selections, slot maps, page placement and V bit
for bit.  The oracle's selections run on the GPU's own float32 scores (both
sides then rank the same values); its R_b runs on its own index, rounded to
bf16 as the index is stored.
"""

import numpy as np
import pytest
import torch

import oracle
from attention_space_retrieval_amd import kvs, workloads as W
from tests.helpers import assert_rel, assert_within_ulp, bits, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 2e-3


def _size(rng, hi):
    """A size in [1, hi], log-uniform, so single-tile and single-chunk cases come up as often as long ones."""
    return min(hi, int(np.exp(rng.uniform(0.0, np.log(hi)))) + 1)


def _forced(rng, N):
    """A protected prefix [0, pi) and a query span [q_s, q_e): mostly at the end of the cache."""
    pi = int(rng.integers(0, min(N, 128) + 1))
    if rng.random() < 0.6:
        q_e = N
        q_s = max(0, N - int(rng.integers(0, 129)))
    else:
        q_s = int(rng.integers(0, N + 1))
        q_e = int(rng.integers(q_s, N + 1))
    return pi, q_s, q_e


@pytest.mark.parametrize("seed", range(16))
def test_rule_turn_random_shapes(seed):
    rng = np.random.default_rng([77, seed])
    L, H_kv, G = int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    H_q, D, N = G * H_kv, int(rng.choice([64, 128])), _size(rng, 6000)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    pi, q_s, q_e = _forced(rng, N)
    print(f"[sweep rule {seed}] L{L} Hq{H_q} Hkv{H_kv} D{D} N{N} {dtype} pi{pi} span[{q_s},{q_e})", flush=True)
    K = W.normal((L, H_kv, N, D), 9000 + seed, W.T_K, dtype, DEV)
    M = W.memory_vectors(L, H_q, D, 9000 + seed, DEV)
    rule = kvs.kvs_rule_score(K, M, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = rule.cpu().numpy()
    want = oracle.rule_score(host(K), host(M), pi, q_s, q_e)
    F = oracle.forced_mask(N, pi, q_s, q_e)
    assert np.all(got[F] == 0.0)
    if (~F).any():
        assert_rel(got[~F], want[~F], RTOL, f"rule score, case {seed}")
        assert abs(got.sum(dtype=np.float64) - L * H_q) <= 1e-4 * L * H_q
    # selection and slot redirect on the GPU's scores, one call
    C = int(rng.integers(0, N + 33))
    slots = torch.from_numpy(rng.permutation(N + 64)[:N].astype(np.int64)).to(DEV)
    dead = int(rng.choice([-1, N + 100]))
    keep, idx, nk, slot_out = kvs.kvs_topk_select_redirect(rule, (0, pi), (q_s, q_e), C, slots, dead)
    torch.cuda.synchronize()
    o_keep, o_idx, o_nk = oracle.topk_select(got, (0, pi), (q_s, q_e), C)
    assert int(nk.item()) == o_nk
    np.testing.assert_array_equal(keep.cpu().numpy().astype(bool), o_keep)
    np.testing.assert_array_equal(idx[:o_nk].cpu().numpy(), o_idx)
    np.testing.assert_array_equal(slot_out.cpu().numpy(),
                                  oracle.slotmap_redirect(slots.cpu().numpy(), o_keep, dead))


@pytest.mark.parametrize("seed", range(12))
def test_window_score_random_shapes(seed):
    rng = np.random.default_rng([78, seed])
    L, H_kv, G = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    H_q, D, N = G * H_kv, int(rng.choice([64, 128])), _size(rng, 3000)
    Wn = _size(rng, 40)
    pi, q_s, q_e = _forced(rng, N)
    print(f"[sweep window {seed}] L{L} Hq{H_q} Hkv{H_kv} D{D} N{N} W{Wn} pi{pi} span[{q_s},{q_e})", flush=True)
    K = W.normal((L, H_kv, N, D), 9100 + seed, W.T_K, "bf16", DEV)
    Qw = W.normal((L, H_q, Wn, D), 9100 + seed, W.T_Q, "bf16", DEV)
    got = kvs.kvs_window_score(K, Qw, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.window_score(host(K), host(Qw), pi, q_s, q_e)
    F = oracle.forced_mask(N, pi, q_s, q_e)
    assert np.all(got[F] == 0.0)
    if (~F).any():
        assert_rel(got[~F], want[~F], RTOL, f"window score, case {seed}")
        assert abs(got.sum(dtype=np.float64) - L * H_q * Wn) <= 1e-4 * L * H_q * Wn


@pytest.mark.parametrize("seed", range(12))
def test_meank_step_random_shapes(seed):
    rng = np.random.default_rng([79, seed])
    L, H_kv, G = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 7))
    H_q, D = G * H_kv, int(rng.choice([64, 128]))
    nB = _size(rng, 300)
    N = 32 * nB - int(rng.integers(0, 32)) if nB > 1 else 32
    Mq = _size(rng, 64)
    sink, recent = int(rng.integers(0, min(nB, 8) + 1)), int(rng.integers(0, min(nB, 16) + 1))
    budget = int(rng.integers(0, nB + 9))
    pos_base, theta = int(rng.integers(0, 1 << 20)), 1e6
    print(f"[sweep meank {seed}] L{L} Hq{H_q} Hkv{H_kv} D{D} N{N} nB{nB} Mq{Mq} sink{sink} recent{recent} "
          f"budget{budget} pos{pos_base}", flush=True)
    K = W.normal((L, H_kv, N, D), 9200 + seed, W.T_K, "bf16", DEV)
    V = W.normal((L, H_kv, N, D), 9200 + seed, W.T_V, "bf16", DEV)
    Q = W.normal((L, H_q, Mq, D), 9200 + seed, W.T_Q, "bf16", DEV)
    # the index, from raw K
    index = kvs.kvs_meank_build(K)
    torch.cuda.synchronize()
    o_index, _ = oracle.meank_build(host(K))
    assert_within_ulp(bits(index), o_index, f"index, case {seed}", atol=1e-5)
    # R_b: the GPU on its index, the oracle on its own, rounded to bf16 as the index is stored
    R = kvs.kvs_meank_score(Q, index, sink, recent)
    torch.cuda.synchronize()
    got = R.cpu().numpy()
    want = oracle.meank_score(host(Q), oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(o_index)), sink, recent)
    Cb = oracle.candidate_blocks(nB, sink, recent)
    assert np.all(got[~Cb] == 0.0)
    if Cb.any():
        assert_rel(got[Cb], want[Cb], RTOL, f"R_b, case {seed}")
        assert abs(got.sum(dtype=np.float64) - Mq) <= 1e-4 * Mq
    # selection on the GPU's R_b, then the scatter of the oracle's selection through a page table
    keep, idx, nk = kvs.kvs_topk_select(R, (0, sink), (nB - recent, nB), budget)
    torch.cuda.synchronize()
    o_sel, _, _ = oracle.meank_select(got, sink, recent, budget)
    n_sel = int(nk.item())
    assert n_sel == len(o_sel)
    np.testing.assert_array_equal(idx[:n_sel].cpu().numpy(), o_sel)
    if n_sel == 0:
        return
    pool_pages = n_sel + int(rng.integers(0, 9))
    pt = W.page_permutation(n_sel, pool_pages, 9200 + seed).to(DEV)
    src_block = torch.from_numpy(o_sel.astype(np.int32)).to(DEV)
    k_pool = torch.full((L, H_kv, 32 * pool_pages, D), -3.0, dtype=torch.bfloat16, device=DEV)
    v_pool = torch.full_like(k_pool, 5.0)
    Kp = torch.nn.functional.pad(K, (0, 0, 0, 32 * nB - N)) if N < 32 * nB else K
    Vp = torch.nn.functional.pad(V, (0, 0, 0, 32 * nB - N)) if N < 32 * nB else V
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kvs.kvs_rerope_scatter(Kp, Vp, src_block, pt, n_sel, pos_base, theta, k_pool, v_pool, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    k0 = np.full((L, H_kv, 32 * pool_pages, D), -3.0)
    v0 = np.full((L, H_kv, 32 * pool_pages, D), 0x40A0, dtype=np.uint16)
    ko, vo = oracle.rerope_scatter(host(Kp), host(Vp), o_sel, pt.cpu().numpy(), pos_base, theta, k0, v0)
    assert_within_ulp(bits(k_pool), ko, f"re-RoPE'd K, case {seed}", atol=1e-6)
    np.testing.assert_array_equal(bits(v_pool), vo)


@pytest.mark.parametrize("seed", range(10))
def test_rule_paged_random_shapes(seed):
    """The rule score read in place from a token-major pool through a seeded slot map, some slots dead
    (-1 or past the pool): against the oracle's paged score."""
    rng = np.random.default_rng([80, seed])
    L, H_kv, G = int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    H_q, D, N = G * H_kv, int(rng.choice([64, 128])), _size(rng, 4000)
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    pool_size = N + int(rng.integers(0, 300))
    pi, q_s, q_e = _forced(rng, N)
    print(f"[sweep paged {seed}] L{L} Hq{H_q} Hkv{H_kv} D{D} N{N} pool{pool_size} {dtype} pi{pi} "
          f"span[{q_s},{q_e})", flush=True)
    pool = W.normal((L, pool_size, H_kv, D), 9300 + seed, W.T_K, dtype, DEV)
    slots = rng.permutation(pool_size)[:N].astype(np.int64)
    n_dead = int(rng.integers(0, min(N, 40) + 1))
    dead_at = rng.choice(N, n_dead, replace=False) if n_dead else np.array([], dtype=np.int64)
    slots[dead_at] = np.where(rng.random(n_dead) < 0.5, -1, pool_size + 7)
    M = W.memory_vectors(L, H_q, D, 9300 + seed, DEV)
    got = kvs.kvs_rule_score_paged(pool, torch.from_numpy(slots).to(DEV), M, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.rule_score_paged(host(pool), slots, host(M), pi, q_s, q_e)
    out = oracle.forced_mask(N, pi, q_s, q_e) | (slots < 0) | (slots >= pool_size)
    np.testing.assert_array_equal(got[out], 0.0)
    if (~out).any():
        assert_rel(got[~out], want[~out], RTOL, f"paged rule score, case {seed}")


@pytest.mark.parametrize("seed", range(10))
def test_working_set_random_sets(seed):
    """Differential working-set update between two seeded selections (retained blocks that keep or
    change rank, incoming and outgoing ones): pages, ranks, released pages, the pool (K within 1 ulp,
    V bit for bit) and every page it must not touch, against the oracle."""
    from tests.test_gpu_meank import _workset_case
    rng = np.random.default_rng([81, seed])
    L, H_kv, D = int(rng.integers(1, 3)), int(rng.integers(1, 6)), int(rng.choice([64, 128]))
    S = _size(rng, 64)
    prev = sorted(rng.choice(S, int(rng.integers(0, S + 1)), replace=False).tolist())
    keep_some = [b for b in prev if rng.random() < 0.6]
    fresh = rng.choice(S, int(rng.integers(0, S + 1)), replace=False).tolist()
    new = sorted(set(keep_some) | set(fresh))
    pool_pages = max(len(prev), len(new), 1) + int(rng.integers(0, 8))
    prev_pages = rng.permutation(pool_pages)[:len(prev)].tolist()
    pos_base, with_v = int(rng.integers(0, 1 << 20)), bool(rng.random() < 0.7)
    print(f"[sweep workset {seed}] L{L} Hkv{H_kv} D{D} blocks{S} pages{pool_pages} prev{len(prev)} "
          f"new{len(new)} v{int(with_v)}", flush=True)
    _workset_case(L, H_kv, D, S, pool_pages, prev, prev_pages, new, pos_base, with_v, 9400 + seed)


@pytest.mark.parametrize("seed", range(6))
def test_rule_score_large_random_shapes(seed):
    """Long caches (10k-100k positions, up to 4 layers and 8 KV heads), where the work-queue fold runs
    thousands of chunks over every resident workgroup: the scores against the oracle, the selection
    on them bit for bit."""
    rng = np.random.default_rng([82, seed])
    L, H_kv, G = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
    H_q, D = G * H_kv, int(rng.choice([64, 128]))
    N = int(np.exp(rng.uniform(np.log(10000), np.log(100000))))
    pi, q_s, q_e = _forced(rng, N)
    print(f"[sweep rule-large {seed}] L{L} Hq{H_q} Hkv{H_kv} D{D} N{N} pi{pi} span[{q_s},{q_e})", flush=True)
    K = W.normal((L, H_kv, N, D), 9500 + seed, W.T_K, "bf16", DEV)
    M = W.memory_vectors(L, H_q, D, 9500 + seed, DEV)
    rule = kvs.kvs_rule_score(K, M, pi, q_s, q_e)
    torch.cuda.synchronize()
    got = rule.cpu().numpy()
    want = oracle.rule_score(host(K), host(M), pi, q_s, q_e)
    F = oracle.forced_mask(N, pi, q_s, q_e)
    assert np.all(got[F] == 0.0)
    assert_rel(got[~F], want[~F], RTOL, f"rule score, large case {seed}")
    assert abs(got.sum(dtype=np.float64) - L * H_q) <= 1e-4 * L * H_q
    C = int(rng.integers(0, N))
    keep, idx, nk = kvs.kvs_topk_select(rule, (0, pi), (q_s, q_e), C)
    torch.cuda.synchronize()
    o_keep, o_idx, o_nk = oracle.topk_select(got, (0, pi), (q_s, q_e), C)
    assert int(nk.item()) == o_nk
    np.testing.assert_array_equal(idx[:o_nk].cpu().numpy(), o_idx)
