"""Rule score, IntentKV Sec. 3.2 Eqs. (3)-(4) (test infrastructure only).

For every layer l and query head h, a softmax over the candidate positions H
of M_t[l,h] . K[l,g(h),j] / sqrt(D) (Eq. 4), summed over all (l, h) into
rule_j (Eq. 3).  The candidate set is H = [0, N) minus the forced set
F = [0, pi) U [q_s, q_e) of Sec. 3.1.

Readings: GQA expands KV head g to the G = H_q / H_kv consecutive query heads
g*G .. g*G+G-1, i.e. g(h) = h // G; forced positions get score 0 (selection
never looks at them).
"""

import math

import numpy as np

from .bf16 import as_f64


def forced_mask(N, pi, q_s, q_e):
    """Boolean [N]: the forced set F = [0, pi) U [q_s, q_e), clipped to [0, N)."""
    F = np.zeros(N, dtype=bool)
    F[: max(0, min(pi, N))] = True
    lo, hi = max(0, q_s), min(N, q_e)
    if hi > lo:
        F[lo:hi] = True
    return F


def rule_score(K, M, pi, q_s, q_e, exclude=None):
    """rule_j for j in [0, N); 0 on the forced set.

    K: [L, H_kv, N, D] post-RoPE keys (float or bf16 bits).
    M: [L, H_q, D] QueryMemory.
    exclude: optional boolean [N]; those positions are not candidates either
    (and score 0), used for positions without a key.
    """
    K = np.asarray(K)
    M = np.asarray(M, dtype=np.float64)
    L, H_kv, N, D = K.shape
    H_q = M.shape[1]
    if M.shape != (L, H_q, D) or H_q % H_kv != 0:
        raise ValueError("shape mismatch between K and M")
    G = H_q // H_kv
    cand = ~forced_mask(N, pi, q_s, q_e)
    if exclude is not None:
        cand &= ~np.asarray(exclude, dtype=bool)
    rule = np.zeros(N, dtype=np.float64)
    if not cand.any():
        return rule
    scale = 1.0 / math.sqrt(D)
    for l in range(L):
        for g in range(H_kv):
            Kc = as_f64(K[l, g])[cand]               # [|H|, D]
            for h in range(g * G, (g + 1) * G):
                s = (Kc @ M[l, h]) * scale            # Eq. (4) logits over H
                a = np.exp(s - s.max())
                a /= a.sum()
                rule[cand] += a                        # Eq. (3)
    return rule


def rule_score_paged(K_pool, slots, M, pi, q_s, q_e):
    """Rule score with K read in place from a paged pool through the slot map.

    IntentKV Sec. 3.1 gives the request's slot map S_r; the layout layer
    (abstract, Sec. 1) keeps survivors in their slots of the paged cache and
    sends dropped positions to a dead slot.  Reading: key row j of KV head g
    in layer l is K_pool[l, S_r[j], g, :] (token-major pool, as SGLang and vLLM
    store it); a position whose slot lies outside the pool has no key, so it
    is not a candidate and scores 0.  Parity unpinned: the pages do not say
    how dead positions enter later scoring.

    K_pool: [L, pool_size, H_kv, D]; slots: [N] integers.
    """
    K_pool = as_f64(K_pool)
    slots = np.asarray(slots, dtype=np.int64)
    L, P, H_kv, D = K_pool.shape
    N = slots.shape[0]
    live = (slots >= 0) & (slots < P)
    K = np.zeros((L, H_kv, N, D), dtype=np.float64)
    K[:, :, live, :] = K_pool[:, slots[live], :, :].transpose(0, 2, 1, 3)
    return rule_score(K, M, pi, q_s, q_e, exclude=~live)


def window_score(K, Qw, pi, q_s, q_e):
    """Window score: SnapKV's window of W query rows, the form IntentKV Sec. 3.2
    says Eq. (3) replaces with a single accumulated query state.

    Reading: for every layer l, query head h and window row w, a softmax over
    the candidate positions H (Sec. 3.1) of Qw[l,h,w] . K[l,g(h),j] / sqrt(D);
    score_j sums them over (l, h, w).  SnapKV's pooling and per-head selection
    are not described by the pages and are left out.  Parity unpinned beyond
    this reading (W = 1 with Qw = M is pinned to the rule score).

    K: [L, H_kv, N, D]; Qw: [L, H_q, W, D] post-RoPE window query rows.
    """
    K = np.asarray(K)
    Qw = as_f64(Qw)
    L, H_kv, N, D = K.shape
    H_q, W = Qw.shape[1], Qw.shape[2]
    if Qw.shape[0] != L or Qw.shape[3] != D or H_q % H_kv != 0:
        raise ValueError("shape mismatch between K and Qw")
    G = H_q // H_kv
    cand = ~forced_mask(N, pi, q_s, q_e)
    score = np.zeros(N, dtype=np.float64)
    if not cand.any() or W == 0:
        return score
    scale = 1.0 / math.sqrt(D)
    for l in range(L):
        for g in range(H_kv):
            Kc = as_f64(K[l, g])[cand]                      # [|H|, D]
            for h in range(g * G, (g + 1) * G):
                S = (Qw[l, h] @ Kc.T) * scale                # [W, |H|]
                S -= S.max(axis=1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(axis=1, keepdims=True)            # softmax over H per window row
                score[cand] += P.sum(axis=0)
    return score
