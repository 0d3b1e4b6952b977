"""QueryMemory update, IntentKV Sec. 3.2 Eq. (2) (test infrastructure only).

M_t = exp(-lambda) * M_{t-1} + Enc(q_t), then M_t is projected to unit length
along the head dimension after every update.  Enc averages the post-RoPE query
rows of the actionable query span.  M has the shape of one post-RoPE query
row, [L, H_q, D].

Readings where the page is silent:
* before the first turn M is zero, so M_0 = Enc(q_0) / ||Enc(q_0)||;
* the recursion carries the stored, already normalised M_{t-1};
* a zero vector stays zero (no direction to project onto);
* lambda = +inf is the page's "query" mode (only the current query counts).
Parity unpinned: the lambda value the paper used is in an appendix that the
page does not contain; callers pass it.
"""

import math

import numpy as np

from .bf16 import as_f64


def enc_span(q_span):
    """Enc(q_t): mean over the span's token rows, per layer and query head.

    q_span: [L, H_q, S, D] post-RoPE query rows (float or bf16 bits).
    Returns float64 [L, H_q, D].
    """
    q = as_f64(q_span)
    if q.ndim != 4 or q.shape[2] == 0:
        raise ValueError("q_span must be [L, H_q, S, D] with S >= 1")
    return q.mean(axis=2)


def qmem_update(q_span, lam, M_prev=None):
    """One QueryMemory step.  M_prev=None means the first turn of a session.

    Returns float64 [L, H_q, D] with every (l, h) row of unit length (or zero).
    """
    enc = enc_span(q_span)
    if M_prev is None:
        M = enc.copy()
    else:
        decay = math.exp(-lam) if lam != math.inf else 0.0
        M = decay * np.asarray(M_prev, dtype=np.float64) + enc
    norm = np.sqrt((M * M).sum(axis=-1, keepdims=True))
    safe = np.where(norm > 0.0, norm, 1.0)
    return np.where(norm > 0.0, M / safe, 0.0)
