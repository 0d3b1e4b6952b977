"""Pins of the oracle to things other than itself.

Invariants fixed by the definitions, closed forms, special cases that reduce
to library routines (torch.softmax in float64, numpy stable argsort, complex
multiplication), and brute force in plain Python loops on tiny inputs.  Each
test names the mistake it would catch.
"""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- QueryMemory

def _qmem_brute(turns, lam):
    """Plain-loop QueryMemory over a list of [L][H][S][D] nested lists."""
    M = None
    for q in turns:
        L, H, S, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
        new = [[[0.0] * D for _ in range(H)] for _ in range(L)]
        for l in range(L):
            for h in range(H):
                for d in range(D):
                    enc = sum(q[l][h][s][d] for s in range(S)) / S
                    prev = 0.0 if M is None else math.exp(-lam) * M[l][h][d]
                    new[l][h][d] = prev + enc
                n = math.sqrt(sum(v * v for v in new[l][h]))
                new[l][h] = [v / n for v in new[l][h]]
        M = new
    return np.array(M)


def test_qmem_brute_force_three_turns():
    r = rng(1)
    turns = [r.standard_normal((2, 3, 4, 5)) for _ in range(3)]
    M = None
    for q in turns:
        M = oracle.qmem_update(q, 0.5, M)
    ref = _qmem_brute([t.tolist() for t in turns], 0.5)
    np.testing.assert_allclose(M, ref, rtol=0, atol=1e-13)


def test_qmem_unit_norm_and_single_turn_closed_form():
    q = rng(2).standard_normal((3, 4, 7, 16))
    M = oracle.qmem_update(q, 0.3, None)
    np.testing.assert_allclose(np.linalg.norm(M, axis=-1), 1.0, atol=1e-14)
    enc = q.sum(axis=2)                       # direction of the mean = direction of the sum
    np.testing.assert_allclose(M, enc / np.linalg.norm(enc, axis=-1, keepdims=True), atol=1e-14)


def test_qmem_query_mode_forgets_history():
    r = rng(3)
    q0, q1 = r.standard_normal((2, 2, 3, 8)), r.standard_normal((2, 2, 3, 8))
    M0 = oracle.qmem_update(q0, math.inf, None)
    M1 = oracle.qmem_update(q1, math.inf, M0)
    np.testing.assert_allclose(M1, oracle.qmem_update(q1, math.inf, None), atol=1e-15)


def test_qmem_single_turn_scale_invariant_and_zero_stays_zero():
    q = rng(4).standard_normal((1, 2, 5, 8))
    np.testing.assert_allclose(oracle.qmem_update(3.7 * q, 0.5), oracle.qmem_update(q, 0.5), atol=1e-14)
    z = np.zeros((1, 1, 2, 4))
    assert np.all(oracle.qmem_update(z, 0.5) == 0.0)


def test_qmem_decay_weight_two_turns():
    # Two turns with orthogonal encodings: the result is proportional to
    # (exp(-lam) * e_a, e_b), which catches exp(+lam) or a dropped decay.
    lam = 0.7
    q0 = np.zeros((1, 1, 1, 2)); q0[..., 0] = 5.0
    q1 = np.zeros((1, 1, 1, 2)); q1[..., 1] = 1.0
    M = oracle.qmem_update(q1, lam, oracle.qmem_update(q0, lam))
    a = math.exp(-lam)
    np.testing.assert_allclose(M[0, 0], np.array([a, 1.0]) / math.hypot(a, 1.0), atol=1e-15)


# ----------------------------------------------------------------- rule score

def _rule_brute(K, M, pi, q_s, q_e):
    L, Hkv, N, D = K.shape
    Hq = M.shape[1]
    G = Hq // Hkv
    H = [j for j in range(N) if not (j < pi or q_s <= j < q_e)]
    rule = [0.0] * N
    for l in range(L):
        for h in range(Hq):
            g = h // G
            logits = {j: sum(M[l, h, d] * K[l, g, j, d] for d in range(D)) / math.sqrt(D) for j in H}
            z = sum(math.exp(v) for v in logits.values())
            for j in H:
                rule[j] += math.exp(logits[j]) / z
    return np.array(rule)


def test_rule_brute_force_gqa_forced():
    r = rng(5)
    K = r.standard_normal((2, 2, 13, 6))
    M = r.standard_normal((2, 4, 6))
    got = oracle.rule_score(K, M, 2, 9, 11)
    np.testing.assert_allclose(got, _rule_brute(K, M, 2, 9, 11), rtol=1e-13, atol=1e-15)


def test_rule_paged_equals_dense_under_any_slot_layout():
    # A pool holding K[l, g, j] at slot perm[j] read through slots = perm gives the dense
    # score exactly: catches a transposed pool index or reading slot j instead of S[j].
    r = rng(14)
    L, Hq, Hkv, N, D, P = 2, 8, 2, 40, 16, 64
    K = r.standard_normal((L, Hkv, N, D))
    M = r.standard_normal((L, Hq, D))
    perm = r.permutation(P)[:N]
    pool = r.standard_normal((L, P, Hkv, D))
    pool[:, perm, :, :] = K.transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(oracle.rule_score_paged(pool, perm, M, 3, 30, 35),
                                  oracle.rule_score(K, M, 3, 30, 35))


def test_rule_paged_dead_slots_brute_force():
    # Positions on the dead slot are no candidates: brute force over the live positions only.
    r = rng(15)
    L, Hq, Hkv, N, D, P = 1, 4, 2, 11, 5, 16
    pool = r.standard_normal((L, P, Hkv, D))
    M = r.standard_normal((L, Hq, D))
    slots = r.permutation(P)[:N].copy()
    slots[[2, 5, 6]] = -1
    got = oracle.rule_score_paged(pool, slots, M, 1, 9, 10)
    live = [j for j in range(N) if slots[j] >= 0 and not (j < 1 or 9 <= j < 10)]
    want = np.zeros(N)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        lg = {j: float(pool[0, slots[j], g] @ M[0, h]) / math.sqrt(D) for j in live}
        z = sum(math.exp(v) for v in lg.values())
        for j in live:
            want[j] += math.exp(lg[j]) / z
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)
    assert got[2] == got[5] == got[6] == 0.0


def test_window_one_row_is_the_rule_score():
    # A window of one row holding M is exactly the rule score (Eq. 3 replaces the window by M).
    r = rng(16)
    K = r.standard_normal((2, 2, 50, 8))
    M = r.standard_normal((2, 4, 8))
    np.testing.assert_allclose(oracle.window_score(K, M[:, :, None, :], 3, 40, 45),
                               oracle.rule_score(K, M, 3, 40, 45), rtol=1e-13, atol=1e-16)


def test_window_brute_force_mass_and_additivity():
    r = rng(17)
    L, Hq, Hkv, N, D, Wn = 1, 4, 2, 12, 5, 3
    K = r.standard_normal((L, Hkv, N, D))
    Qw = r.standard_normal((L, Hq, Wn, D))
    got = oracle.window_score(K, Qw, 2, 8, 10)
    H = [j for j in range(N) if not (j < 2 or 8 <= j < 10)]
    want = np.zeros(N)
    for h in range(Hq):
        for w in range(Wn):
            lg = {j: float(Qw[0, h, w] @ K[0, h // 2, j]) / math.sqrt(D) for j in H}
            z = sum(math.exp(v) for v in lg.values())
            for j in H:
                want[j] += math.exp(lg[j]) / z
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-16)
    assert abs(got.sum() - L * Hq * Wn) < 1e-12                  # each row's softmax sums to one
    split = oracle.window_score(K, Qw[:, :, :1], 2, 8, 10) + oracle.window_score(K, Qw[:, :, 1:], 2, 8, 10)
    np.testing.assert_allclose(got, split, rtol=1e-13)


def test_rule_mass_and_forced_zero():
    r = rng(6)
    L, Hq, Hkv, N, D = 3, 8, 2, 200, 16
    K = r.standard_normal((L, Hkv, N, D))
    M = r.standard_normal((L, Hq, D))
    rule = oracle.rule_score(K, M, 10, 150, 170)
    F = oracle.forced_mask(N, 10, 150, 170)
    assert np.all(rule[F] == 0.0) and np.all(rule[~F] > 0.0)
    assert abs(rule.sum() - L * Hq) < 1e-11          # each softmax sums to one


def test_rule_identical_rows_uniform_and_shift_invariant():
    r = rng(7)
    L, Hq, Hkv, N, D = 2, 4, 2, 50, 8
    row = r.standard_normal(D)
    K = np.broadcast_to(row, (L, Hkv, N, D)).copy()
    M = r.standard_normal((L, Hq, D))
    rule = oracle.rule_score(K, M, 3, 40, 45)
    nH = N - 3 - 5
    F = oracle.forced_mask(N, 3, 40, 45)
    np.testing.assert_allclose(rule[~F], L * Hq / nH, rtol=1e-13)
    # softmax is invariant to adding the same vector to every key of a head
    K2 = r.standard_normal((L, Hkv, N, D))
    shifted = K2 + r.standard_normal((L, Hkv, 1, D))
    np.testing.assert_allclose(oracle.rule_score(shifted, M, 3, 40, 45),
                               oracle.rule_score(K2, M, 3, 40, 45), rtol=1e-11)


def test_rule_single_head_is_torch_softmax():
    r = rng(8)
    N, D = 64, 32
    K = r.standard_normal((1, 1, N, D))
    M = r.standard_normal((1, 1, D))
    ref = torch.softmax(torch.from_numpy(K[0, 0] @ M[0, 0] / math.sqrt(D)), dim=0).numpy()
    np.testing.assert_allclose(oracle.rule_score(K, M, 0, N, N), ref, rtol=1e-13)


def test_rule_gqa_equals_explicit_expansion():
    r = rng(9)
    L, Hq, Hkv, N, D = 2, 6, 2, 40, 8
    K = r.standard_normal((L, Hkv, N, D))
    M = r.standard_normal((L, Hq, D))
    Kexp = torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=1)       # [L, Hq, N, D]
    logits = torch.einsum("lhnd,lhd->lhn", Kexp, torch.from_numpy(M)) / math.sqrt(D)
    mask = torch.from_numpy(oracle.forced_mask(N, 4, 30, 33))
    logits[..., mask] = -math.inf
    ref = torch.softmax(logits, dim=-1).sum(dim=(0, 1)).numpy()
    np.testing.assert_allclose(oracle.rule_score(K, M, 4, 30, 33), ref, rtol=1e-12, atol=1e-300)


def test_rule_all_forced_is_zero():
    K = rng(10).standard_normal((1, 1, 8, 4))
    M = rng(11).standard_normal((1, 2, 4))
    assert np.all(oracle.rule_score(K, M, 8, 0, 0) == 0.0)


# ----------------------------------------------------------------- top-k

def _topk_brute(score, forced, C):
    n = len(score)
    F = [j for j in range(n) if forced[j]]
    H = [j for j in range(n) if not forced[j]]
    c_star = min(max(0, C - len(F)), len(H))
    best = None
    for comb in itertools.combinations(H, c_star):          # ascending tuples
        total = sum(score[j] for j in comb)
        key = (-total, comb)                                 # max sum, then lexicographically smallest
        if best is None or key < best:
            best = key
    return sorted(F + list(best[1]))


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_with_ties(seed):
    r = rng(100 + seed)
    n = int(r.integers(1, 13))
    score = r.integers(0, 4, size=n).astype(np.float64) / 4.0    # many exact ties
    f0 = (0, int(r.integers(0, 3)))
    b = int(r.integers(0, n + 1))
    f1 = (b, b + int(r.integers(0, 3)))
    C = int(r.integers(0, n + 3))
    forced = np.zeros(n, bool)
    forced[f0[0]:f0[1]] = True
    forced[max(0, f1[0]):min(n, f1[1])] = True
    keep, idx, nk = oracle.topk_select(score, f0, f1, C)
    assert idx.tolist() == _topk_brute(score.tolist(), forced.tolist(), C)
    assert nk == forced.sum() + min(max(0, C - forced.sum()), n - forced.sum())


def test_topk_matches_stable_argsort_and_invariants():
    r = rng(200)
    n = 5000
    score = np.round(r.standard_normal(n), 2)                 # ties
    keep, idx, nk = oracle.topk_select(score, (0, 17), (4900, 5000), 1200)
    forced = np.zeros(n, bool); forced[:17] = True; forced[4900:] = True
    cand = np.flatnonzero(~forced)
    order = cand[np.argsort(-score[cand], kind="stable")]     # stable: equal scores keep index order
    expect = np.sort(np.concatenate([np.flatnonzero(forced), order[: 1200 - forced.sum()]]))
    np.testing.assert_array_equal(idx, expect)
    assert np.all(np.diff(idx) > 0) and keep[forced].all() and nk == 1200


def test_topk_all_equal_keeps_lowest_indices_and_nan_last():
    keep, idx, _ = oracle.topk_select(np.ones(20), (0, 2), (18, 20), 7)
    assert idx.tolist() == [0, 1, 2, 3, 4, 18, 19]             # |F| = 4, C* = 3: lowest candidates
    s = np.array([np.nan, -np.inf, 0.0, -0.0, 1.0])
    _, idx, _ = oracle.topk_select(s, (0, 0), (0, 0), 4)
    assert idx.tolist() == [1, 2, 3, 4]                         # NaN ranks below -inf; -0 ties +0
    _, idx, _ = oracle.topk_select(s, (0, 0), (0, 0), 2)
    assert idx.tolist() == [2, 4]                               # +0 (idx 2) and -0 tie: lower index


def test_slotmap_redirect_invariants():
    r = rng(300)
    N = 1000
    slots = r.permutation(N).astype(np.int64) + 5000
    keep, idx, nk = oracle.topk_select(r.random(N), (0, 16), (980, 1000), 256)
    out = oracle.slotmap_redirect(slots, keep, -1)
    np.testing.assert_array_equal(out[keep], slots[keep])        # survivors keep their slot
    assert (out == -1).sum() == N - nk and np.all(out[~keep] == -1)


# ----------------------------------------------------------------- RoPE

def test_rope_identity_norm_inverse():
    r = rng(400)
    x = r.standard_normal((3, 50, 128))
    pos = r.integers(0, 1 << 20, size=50)
    np.testing.assert_array_equal(oracle.rope_rotate(x, np.zeros(50, int), 1e6), x)
    y = oracle.rope_rotate(x, pos, 1e6)
    pair_norm = lambda v: v[..., :64] ** 2 + v[..., 64:] ** 2
    np.testing.assert_allclose(pair_norm(y), pair_norm(x), rtol=1e-12)
    np.testing.assert_allclose(oracle.rope_rotate(y, pos, 1e6, inverse=True), x, atol=1e-12)


def test_rope_complex_formulation():
    r = rng(401)
    D = 64
    x = r.standard_normal((20, D))
    pos = r.integers(0, 1 << 20, size=20)
    y = oracle.rope_rotate(x, pos, 1e6)
    z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(
        1j * pos[:, None] * (1e6 ** (-np.arange(0, D, 2) / D))[None, :])
    np.testing.assert_allclose(y[:, : D // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, D // 2:], z.imag, atol=1e-12)


def test_rope_relative_position():
    r = rng(402)
    q, k = r.standard_normal((1, 128)), r.standard_normal((1, 128))
    for m, n in [(3, 10), (1000, 70000), (524288, 1048575)]:
        lhs = (oracle.rope_rotate(q, [m], 1e6) * oracle.rope_rotate(k, [n], 1e6)).sum()
        rhs = (q * oracle.rope_rotate(k, [n - m], 1e6)).sum()
        assert abs(lhs - rhs) < 1e-9


# ----------------------------------------------------------------- Mean-K

def _meank_score_brute(Q, index, n_sink, n_recent):
    L, Hq, Mq, D = Q.shape
    Hkv, nB = index.shape[1], index.shape[2]
    G = Hq // Hkv
    C = [b for b in range(nB) if n_sink <= b < nB - n_recent]
    R = [0.0] * nB
    for l in range(L):
        for h in range(Hq):
            for m in range(Mq):
                lg = [sum(Q[l, h, m, d] * index[l, h // G, b, d] for d in range(D)) / math.sqrt(D) for b in C]
                z = sum(math.exp(v) for v in lg)
                for b, v in zip(C, lg):
                    R[b] += math.exp(v) / z
    return np.array(R) / (L * Hq)


def test_meank_score_brute_force():
    r = rng(500)
    Q = r.standard_normal((2, 4, 3, 6))
    index = r.standard_normal((2, 2, 9, 6))
    np.testing.assert_allclose(oracle.meank_score(Q, index, 2, 3),
                               _meank_score_brute(Q, index, 2, 3), rtol=1e-13, atol=1e-16)


def test_meank_score_mass_uniform_and_empty():
    r = rng(501)
    L, Hq, Hkv, Mq, nB, D = 2, 6, 3, 11, 40, 16
    Q = r.standard_normal((L, Hq, Mq, D))
    index = r.standard_normal((L, Hkv, nB, D))
    R = oracle.meank_score(Q, index, 4, 6)
    C = oracle.candidate_blocks(nB, 4, 6)
    assert abs(R.sum() - Mq) < 1e-11 and np.all(R[~C] == 0) and np.all(R[C] > 0)
    flat = np.broadcast_to(r.standard_normal(D), (L, Hkv, nB, D))
    np.testing.assert_allclose(oracle.meank_score(Q, flat, 4, 6)[C], Mq / C.sum(), rtol=1e-13)
    assert np.all(oracle.meank_score(Q, index, 20, 20) == 0.0)


def test_meank_score_block1_is_torch_softmax_colsum():
    r = rng(502)
    Mq, N, D = 9, 30, 8
    Q = r.standard_normal((1, 1, Mq, D))
    K = r.standard_normal((1, 1, N, D))
    index, _ = oracle.meank_build(K, block=1)
    ref = torch.softmax(torch.from_numpy(Q[0, 0] @ K[0, 0].T / math.sqrt(D)), dim=-1).sum(0).numpy()
    np.testing.assert_allclose(oracle.meank_score(Q, index, 0, 0), ref, rtol=1e-13)


def test_meank_score_gqa_equals_explicit_expansion():
    r = rng(503)
    L, Hq, Hkv, Mq, nB, D = 2, 4, 2, 5, 12, 8
    Q = r.standard_normal((L, Hq, Mq, D))
    index = r.standard_normal((L, Hkv, nB, D))
    idx = torch.from_numpy(index).repeat_interleave(Hq // Hkv, dim=1)[:, :, 1:10]   # C = [1, 10)
    P = torch.softmax(torch.from_numpy(Q) @ idx.transpose(-1, -2) / math.sqrt(D), dim=-1)
    ref = np.zeros(nB)
    ref[1:10] = P.sum(dim=(0, 1, 2)).numpy() / (L * Hq)
    np.testing.assert_allclose(oracle.meank_score(Q, index, 1, 2), ref, rtol=1e-12)


def test_meank_build_brute_constant_linear_partial():
    r = rng(504)
    K = r.standard_normal((2, 3, 70, 4))
    index, _ = oracle.meank_build(K, block=32)
    assert index.shape == (2, 3, 3, 4)
    for l, g, b in itertools.product(range(2), range(3), range(3)):
        rows = range(32 * b, min(70, 32 * b + 32))
        for d in range(4):
            assert abs(index[l, g, b, d] - sum(K[l, g, i, d] for i in rows) / len(rows)) < 1e-14
    c = np.full((1, 1, 64, 4), 2.5)
    assert np.all(oracle.meank_build(c)[0] == 2.5)
    K2 = r.standard_normal(K.shape)
    np.testing.assert_allclose(oracle.meank_build(2 * K - 3 * K2)[0],
                               2 * oracle.meank_build(K)[0] - 3 * oracle.meank_build(K2)[0], atol=1e-13)


def test_meank_build_derope_round_trip_and_position_independence():
    r = rng(505)
    raw = r.standard_normal((2, 2, 96, 32))
    for pos0 in (0, 12345, 1000000):
        post = oracle.rope_rotate(raw, pos0 + np.arange(96), 1e6)
        idx, raw_back = oracle.meank_build(post, k_is_rope=True, pos0=pos0, theta=1e6)
        np.testing.assert_allclose(raw_back, raw, atol=1e-10)
        np.testing.assert_allclose(idx, oracle.meank_build(raw)[0], atol=1e-10)


def _append_all(post, pos0, chunks, theta=1e6, cap=None):
    """Run meank_append over consecutive chunks; return (stage bits, index dict block -> mean)."""
    L, H, N, D = post.shape
    stage = np.zeros((L, H, cap or N, D), dtype=np.uint16)
    index, t0 = {}, 0
    for n in chunks:
        stage, b0, means = oracle.meank_append(post[:, :, t0:t0 + n], t0, pos0, theta, stage)
        for i in range(means.shape[2]):
            index[b0 + i] = means[:, :, i]
        t0 += n
    return stage, index


def test_meank_append_stage_is_derope_of_the_chunk():
    # Catches a wrong position offset for chunk rows (pos0 + i instead of pos0 + t0 + i)
    # or a wrong rotation direction: the stage must be the a6 de-RoPE of the same keys.
    r = rng(507)
    post = oracle.f64_to_bf16_bits(r.standard_normal((2, 2, 150, 32)))
    for pos0 in (0, 999000):
        stage, _ = _append_all(post, pos0, [37, 1, 64, 48])
        _, raw = oracle.meank_build(post, k_is_rope=True, pos0=pos0, theta=1e6)
        np.testing.assert_array_equal(stage, oracle.f64_to_bf16_bits(raw))


def test_meank_append_index_is_raw_build_of_the_stage():
    # Catches dropped earlier rows of a partially filled block, a wrong divisor for a
    # partial block, or averaging unrounded instead of staged values.
    r = rng(508)
    post = oracle.f64_to_bf16_bits(r.standard_normal((1, 3, 200, 16)))
    for chunks in ([200], [5, 27, 32, 100, 36], [31, 2, 31, 136], [64, 0, 136]):
        stage, index = _append_all(post, 777, chunks)
        want, _ = oracle.meank_build(oracle.bf16_bits_to_f64(stage))
        assert sorted(index) == list(range(want.shape[2]))
        for b, m in index.items():
            np.testing.assert_allclose(m, want[:, :, b], rtol=0, atol=1e-15)


def test_meank_append_round_trip_recovers_raw():
    # RoPE applied forward (pinned by complex multiplication) then removed by the
    # append gives the raw keys back to bf16 rounding.
    r = rng(509)
    raw = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(r.standard_normal((2, 1, 70, 64))))
    pos0 = 123456
    post = oracle.f64_to_bf16_bits(oracle.rope_rotate(raw, pos0 + np.arange(70), 1e6))
    stage, _ = _append_all(post, pos0, [33, 37])
    got = oracle.bf16_bits_to_f64(stage)
    assert np.max(np.abs(got - raw)) <= 2 * 2.0 ** -8 * np.max(np.abs(raw))


def _pool_from_scatter(raw_k, raw_v, blocks, pages, pool_pages, pos_base, theta=1e6):
    L, H, _, D = raw_k.shape
    kp = np.zeros((L, H, 32 * pool_pages, D))
    vp = np.zeros((L, H, 32 * pool_pages, D))
    return oracle.rerope_scatter(raw_k, raw_v, blocks, pages, pos_base, theta, kp, vp)


def test_workset_empty_previous_is_the_scatter():
    # With nothing resident the update is the plain re-RoPE scatter onto pages 0, 1, ...
    r = rng(510)
    raw_k, raw_v = r.standard_normal((2, 2, 32 * 20, 16)), r.standard_normal((2, 2, 32 * 20, 16))
    new = [1, 4, 5, 11, 19]
    kp, vp = np.zeros((2, 2, 32 * 8, 16)), np.zeros((2, 2, 32 * 8, 16))
    k, v, pages, old_rank, out = oracle.working_set_update(raw_k, raw_v, [], [], new, 64, 1e6, kp, vp)
    ks, vs = oracle.rerope_scatter(raw_k, raw_v, new, None, 64, 1e6, kp, vp)
    assert pages.tolist() == [0, 1, 2, 3, 4] and (old_rank == -1).all() and len(out) == 0
    np.testing.assert_array_equal(k, ks)
    np.testing.assert_array_equal(v, vs)


def test_workset_moved_blocks_match_rope_at_new_position():
    # A retained block whose compact index moved must equal raw K RoPE'd at the new compact
    # position (KVMEM, "Engineering and cost ...": raw K is the reconstruction authority):
    # catches a block left at its old positions, a rotation by the delta in blocks rather
    # than tokens, or the wrong sign.
    r = rng(511)
    raw_k, raw_v = r.standard_normal((1, 2, 32 * 30, 32)), r.standard_normal((1, 2, 32 * 30, 32))
    prev, prev_pages = [2, 3, 7, 10, 15, 21], [5, 0, 7, 2, 9, 4]
    k0, v0 = _pool_from_scatter(raw_k, raw_v, prev, prev_pages, 12, 100)
    new = [0, 3, 7, 12, 13, 15, 29]
    k, v, pages, old_rank, out = oracle.working_set_update(raw_k, raw_v, prev, prev_pages, new, 100, 1e6, k0, v0)
    want_k, want_v = oracle.rerope_scatter(raw_k, raw_v, new, pages, 100, 1e6, k0, v0)
    for rr, p in enumerate(pages):
        rows = slice(32 * p, 32 * p + 32)
        np.testing.assert_allclose(k[:, :, rows], want_k[:, :, rows], atol=1e-10)
        np.testing.assert_array_equal(v[:, :, rows], want_v[:, :, rows])


def test_workset_chain_of_updates_has_no_drift():
    # Several steps in a row, the pool rounded to bf16 after each one as the library stores it:
    # the final pool equals one re-RoPE scatter of the final selection from raw K onto the final
    # pages, bit for bit.  Rotating a moved block's stored bf16 copy by its position delta would
    # round once more per move and fail this.
    r = rng(513)
    L, H, D, src_blocks, pool, pos_base, theta = 1, 2, 16, 60, 24, 0, 1e6
    raw_k = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(r.standard_normal((L, H, 32 * src_blocks, D)) * 4))
    raw_v = oracle.f64_to_bf16_bits(r.standard_normal((L, H, 32 * src_blocks, D)))
    prev = sorted(r.choice(src_blocks, 12, replace=False).tolist())
    prev_pages = r.permutation(pool)[:12].tolist()
    k, v = oracle.rerope_scatter(raw_k, raw_v, prev, prev_pages, pos_base, theta, np.zeros((L, H, 32 * pool, D)),
                                 np.zeros((L, H, 32 * pool, D), np.uint16))
    k = oracle.f64_to_bf16_bits(k)
    n_moved = 0
    for step in range(8):
        keep = [b for b in prev if r.random() < 0.7]
        new = sorted(set(keep) | set(r.choice(src_blocks, 6, replace=False).tolist()))[:16]
        kf, v, pages, old_rank, _ = oracle.working_set_update(raw_k, raw_v, prev, prev_pages, new, pos_base, theta,
                                                              k, v)
        k = oracle.f64_to_bf16_bits(kf)
        n_moved += sum(1 for i, rr in enumerate(old_rank) if rr >= 0 and rr != i)
        prev, prev_pages = new, pages.tolist()
    assert n_moved >= 8
    ks, vs = oracle.rerope_scatter(raw_k, raw_v, prev, prev_pages, pos_base, theta, np.zeros((L, H, 32 * pool, D)),
                                   np.zeros((L, H, 32 * pool, D), np.uint16))
    for p in prev_pages:
        rows = slice(32 * p, 32 * p + 32)
        np.testing.assert_array_equal(k[:, :, rows], oracle.f64_to_bf16_bits(ks[:, :, rows]))
        np.testing.assert_array_equal(v[:, :, rows], vs[:, :, rows])


def test_workset_classes_pages_and_untouched_rows():
    # Brute-force set algebra for the classes; free pages go out in ascending order;
    # pages of unmoved retained blocks and of outgoing blocks are left bit-identical.
    r = rng(512)
    for trial in range(20):
        pool = 40
        prev = sorted(r.choice(100, size=r.integers(0, 20), replace=False).tolist())
        prev_pages = r.permutation(pool)[:len(prev)].tolist()
        new = sorted(r.choice(100, size=r.integers(0, 25), replace=False).tolist())
        pages, old_rank, out = oracle.working_set_diff(prev, prev_pages, new, pool)
        retained = set(prev) & set(new)
        assert {b for b, i in zip(new, old_rank) if i >= 0} == retained
        assert len(out) == len(set(prev) - set(new))
        assert len(set(pages.tolist())) == len(new) and all(0 <= p < pool for p in pages)
        held = {prev_pages[prev.index(b)] for b in retained}
        free = sorted(set(range(pool)) - held)
        inc_pages = [int(p) for p, i in zip(pages, old_rank) if i < 0]
        assert inc_pages == free[:len(inc_pages)]
        for b, p, i in zip(new, pages, old_rank):
            if i >= 0:
                assert p == prev_pages[prev.index(b)]
    raw_k = r.standard_normal((1, 1, 32 * 10, 8))
    prev, prev_pages = [1, 2, 6], [3, 1, 0]
    k0 = r.standard_normal((1, 1, 32 * 6, 8))
    v0 = r.standard_normal((1, 1, 32 * 6, 8))
    new = [1, 2, 8]          # 1, 2 keep ranks 0, 1; 6 goes out and its page 0 takes 8
    k, v, pages, _, out = oracle.working_set_update(raw_k, raw_k, prev, prev_pages, new, 0, 1e6, k0, v0)
    for p in (3, 1, 2, 4, 5):
        np.testing.assert_array_equal(k[:, :, 32 * p:32 * p + 32], k0[:, :, 32 * p:32 * p + 32])
        np.testing.assert_array_equal(v[:, :, 32 * p:32 * p + 32], v0[:, :, 32 * p:32 * p + 32])
    assert out.tolist() == [0] and pages.tolist() == [3, 1, 0]


def _meank_select_brute(R, n_sink, n_recent, budget, free_pages, pos_base):
    """KVMEM, "Design and trade-offs ... Mean-K": the sink and recent blocks are always kept and the
    rest of the budget goes to the blocks of largest R_b; the selection is laid out in ascending block
    order ("Engineering and cost ...": compact logical order), logical block r on the r-th free page
    (page r when there is no free list) at positions pos_base + 32 r ... +31.  Written as an exhaustive
    search: among all candidate subsets of the remaining budget, the one of largest R sum, the
    lexicographically smallest among equals."""
    nB = len(R)
    forced = [b for b in range(nB) if b < n_sink or b >= nB - n_recent]
    cand = [b for b in range(nB) if b not in forced]
    k = min(max(0, budget - len(forced)), len(cand))
    best = None
    for comb in itertools.combinations(cand, k):
        key = (-sum(R[b] for b in comb), comb)
        if best is None or key < best:
            best = key
    keep = sorted(forced + list(best[1]))
    dst = [free_pages[r] if free_pages is not None else r for r in range(len(keep))]
    return keep, dst, [pos_base + 32 * r for r in range(len(keep))]


def _meank_select_cases():
    r = rng(520)
    for trial in range(60):
        nB = int(r.integers(1, 15))
        R = (r.integers(0, 5, size=nB) / 4.0).tolist()             # exact ties
        n_sink, n_recent = int(r.integers(0, 4)), int(r.integers(0, 5))  # sink and recent may overlap
        budget = int(r.integers(0, nB + 3))
        free = r.permutation(nB + 6).tolist() if trial % 2 else None
        yield R, n_sink, n_recent, budget, free, int(r.integers(0, 5000))


def _check_meank_select(select):
    """Every case against the brute force, plus the properties the page fixes."""
    for R, n_sink, n_recent, budget, free, pos_base in _meank_select_cases():
        keep, dst, pos = select(np.array(R), n_sink, n_recent, budget, free, pos_base)
        want = _meank_select_brute(R, n_sink, n_recent, budget, free, pos_base)
        assert [list(map(int, keep)), list(map(int, dst)), list(map(int, pos))] == [list(w) for w in want], \
            (R, n_sink, n_recent, budget, free, pos_base)
        nB = len(R)
        forced = {b for b in range(nB) if b < n_sink or b >= nB - n_recent}
        assert forced <= set(int(b) for b in keep)
        assert len(keep) == len(forced) + min(max(0, budget - len(forced)), nB - len(forced))
        assert all(a < b for a, b in zip(keep, keep[1:]))


def test_meank_select_brute_force_page_table_and_positions():
    _check_meank_select(lambda R, s, rc, b, fp, pb: oracle.meank_select(R, s, rc, b, fp, pb))


def _select_variant(R, n_sink, n_recent, budget, free, pos_base, recent=True, inclusive=True, pages=True,
                    shift=0):
    """meank_select with one deliberate mistake (for the test below)."""
    nB = len(R)
    f1 = (nB - n_recent, nB) if recent else (nB, nB)
    n_forced = len(set(range(min(n_sink, nB))) | set(range(max(0, nB - n_recent), nB)))
    _, keep, nk = oracle.topk_select(R, (0, n_sink), f1, budget if inclusive else budget + n_forced)
    dst = np.asarray(free)[:nk] if (free is not None and pages) else np.arange(nk)
    return keep, dst, pos_base + 32 * (np.arange(nk) + shift)


@pytest.mark.parametrize("mistake", [dict(recent=False), dict(inclusive=False), dict(pages=False), dict(shift=1)])
def test_meank_select_pin_catches_planted_mistakes(mistake):
    # recent blocks not forced; budget read as excluding the sink and recent blocks; the free list
    # ignored; positions one block off.  The pin must reject each, and accept the unchanged variant.
    _check_meank_select(lambda *a: _select_variant(*a))
    with pytest.raises(AssertionError):
        _check_meank_select(lambda *a: _select_variant(*a, **mistake))


def test_meank_planted_evidence_is_selected():
    # Blocks whose raw K is shifted along a direction the queries share must win.
    r = rng(506)
    L, Hq, Hkv, Mq, N, D = 2, 4, 2, 16, 32 * 64, 32
    u = r.standard_normal(D); u /= np.linalg.norm(u)
    K = r.standard_normal((L, Hkv, N, D))
    planted = [9, 20, 33, 41]
    for b in planted:
        K[:, :, 32 * b: 32 * b + 32, :] += 3.0 * u
    Q = r.standard_normal((L, Hq, Mq, D)) + 4.0 * u
    index, _ = oracle.meank_build(K)
    R = oracle.meank_score(Q, index, 4, 8)
    keep_idx, _, _ = oracle.meank_select(R, 4, 8, 4 + 8 + len(planted))
    assert set(planted) <= set(keep_idx.tolist())


# ----------------------------------------------------------------- bf16

def test_bf16_round_trip_and_rne():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    x = oracle.bf16_bits_to_f64(bits)
    finite = np.isfinite(x)
    back = oracle.f64_to_bf16_bits(x[finite])
    # +0/-0 and every finite pattern round-trip exactly
    np.testing.assert_array_equal(back, bits[finite])
    # agree with torch's float32 -> bf16 RNE on values exact in float32
    v = np.random.default_rng(600).standard_normal(100000).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(v.astype(np.float64)), t)
