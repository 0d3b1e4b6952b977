"""Mean-K index and block relevance R_b (test infrastructure only).

KVMEM, section "Design and trade-offs: step-level attention trigger and
Mean-K model-native retrieval".  Both display equations were lost when the
page was extracted; what survives is the prose and the symbol glossary.  The
readings taken from that prose:

* Mean-K index: for every block b of 32 tokens, layer l and KV head g, the
  arithmetic mean of the position-free (RoPE-removed) keys k~_{l,i,g} over the
  block's tokens -- one vector per block, layer and KV head.  A partial last
  block averages over the tokens it has.
* R_b: for each layer l, query head h and query token m, a softmax over the
  candidate blocks C of q_{l,m,h} . kbar_{l,g(h),b} / sqrt(d), with the
  position-free query q; these are summed over query tokens m and averaged
  over the participating (layer, head) pairs -- all L * H_q of them.
* C = all blocks minus the sink and recent blocks, which are kept regardless.
  R_b = 0 for those forced blocks.
Parity unpinned: whether only a subset of layers votes, and whether the
softmax runs over all history blocks instead of C (the page does not say).
"""

import math

import numpy as np

from .bf16 import as_f64
from .rope import rope_rotate


def meank_build(K, block=32, k_is_rope=False, pos0=0, theta=1e6):
    """Mean-K index, float64 [L, H_kv, ceil(N/block), D].

    K: [L, H_kv, N, D] keys.  With k_is_rope the keys carry RoPE at positions
    pos0 .. pos0+N-1 and it is removed first; otherwise K is already raw.
    Returns (index, raw_k) where raw_k is the RoPE-removed K (or K itself).
    """
    K = as_f64(K)
    L, H_kv, N, D = K.shape
    if k_is_rope:
        raw = rope_rotate(K, pos0 + np.arange(N), theta, inverse=True)
    else:
        raw = K
    nB = -(-N // block)
    index = np.zeros((L, H_kv, nB, D), dtype=np.float64)
    for b in range(nB):
        lo, hi = b * block, min(N, (b + 1) * block)
        index[:, :, b, :] = raw[:, :, lo:hi, :].mean(axis=2)
    return index, raw


def candidate_blocks(nB, n_sink, n_recent):
    """Boolean [nB]: the candidate set C = blocks that are neither sink nor recent."""
    c = np.ones(nB, dtype=bool)
    c[: max(0, min(n_sink, nB))] = False
    lo = max(0, nB - n_recent)
    c[lo:] = False
    return c


def meank_score(Q, index, n_sink, n_recent):
    """R_b for every block, float64 [nB]; 0 on sink and recent blocks.

    Q: [L, H_q, Mq, D] position-free query vectors; index: [L, H_kv, nB, D].
    """
    Q = np.asarray(Q)
    index = np.asarray(index)
    L, H_q, Mq, D = Q.shape
    _, H_kv, nB, _ = index.shape
    if index.shape[0] != L or index.shape[3] != D or H_q % H_kv != 0:
        raise ValueError("shape mismatch between Q and index")
    G = H_q // H_kv
    cand = candidate_blocks(nB, n_sink, n_recent)
    R = np.zeros(nB, dtype=np.float64)
    if not cand.any() or Mq == 0:
        return R
    scale = 1.0 / math.sqrt(D)
    for l in range(L):
        for g in range(H_kv):
            kb = as_f64(index[l, g])[cand]              # [|C|, D]
            for h in range(g * G, (g + 1) * G):
                S = (as_f64(Q[l, h]) @ kb.T) * scale    # [Mq, |C|]
                S -= S.max(axis=1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(axis=1, keepdims=True)       # softmax over C, per query token
                R[cand] += P.sum(axis=0)                # summed over query tokens
    return R / (L * H_q)                                # averaged over (layer, head)
