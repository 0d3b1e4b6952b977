"""Budgeted top-k with a forced set, and the slot-map redirect (test infrastructure only).

IntentKV Sec. 3.1 Eq. (1): with forced set F, remaining budget
C* = max(0, C - |F|) and candidates H = [0, n) \\ F, the kept set is
F U (the C* candidates of largest score).  KVMEM's selection (section "Design
and trade-offs ... Mean-K") is the same rule with F = sink blocks U recent
blocks and C = the block budget.

Eq. (1)'s argmax is not unique when scores tie at the threshold.  The reading
used here: larger score first, equal scores -> lower index first.  NaN ranks
below every number; -0.0 equals +0.0.
"""

import numpy as np


def _range_mask(n, begin, end):
    m = np.zeros(n, dtype=bool)
    lo, hi = max(0, begin), min(n, end)
    if hi > lo:
        m[lo:hi] = True
    return m


def topk_select(score, f0, f1, C):
    """Return (keep_mask bool [n], keep_idx int64 ascending, n_kept).

    score: [n] float scores (compared as given; float32 inputs compare exactly).
    f0, f1: (begin, end) half-open forced ranges, clipped to [0, n).
    C: total budget including the forced positions.
    """
    s = np.asarray(score, dtype=np.float64)
    n = s.shape[0]
    forced = _range_mask(n, *f0) | _range_mask(n, *f1)
    cand = np.flatnonzero(~forced)
    c_star = max(0, C - int(forced.sum()))
    cs = s[cand]
    is_nan = np.isnan(cs)
    neg = np.where(is_nan, 0.0, -cs)
    order = np.lexsort((cand, neg, is_nan))     # primary: not-NaN first, then -score, then index
    chosen = cand[order[:c_star]]
    keep = forced.copy()
    keep[chosen] = True
    keep_idx = np.flatnonzero(keep)
    return keep, keep_idx, int(keep_idx.size)


def slotmap_redirect(slot, keep_mask, dead_slot):
    """IntentKV layout layer: dropped positions point at the dead slot, survivors keep theirs."""
    slot = np.asarray(slot, dtype=np.int64)
    return np.where(np.asarray(keep_mask, dtype=bool), slot, np.int64(dead_slot))


def meank_select(R, n_sink, n_recent, budget, free_pages=None, pos_base=0, block=32):
    """KVMEM selection plus execution-view page table.

    Sink blocks [0, n_sink) and recent blocks [nB - n_recent, nB) are always
    kept; the rest of the budget goes to the largest R_b.  The selected blocks
    are laid out in ascending original order (the compact logical order);
    logical block r lands on physical page free_pages[r] (identity when None)
    and covers positions pos_base + block*r ... + block - 1.

    Returns (keep_idx, dst_pages, first_positions).
    """
    nB = len(R)
    _, keep_idx, n_kept = topk_select(R, (0, n_sink), (nB - n_recent, nB), budget)
    if free_pages is None:
        dst = np.arange(n_kept, dtype=np.int64)
    else:
        dst = np.asarray(free_pages, dtype=np.int64)[:n_kept]
    first_pos = pos_base + block * np.arange(n_kept, dtype=np.int64)
    return keep_idx, dst, first_pos
