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

from .bf16 import as_f64, bf16_bits_to_f64, f64_to_bf16_bits
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


def meank_append(k_chunk, t0, pos0, theta, stage, block=32):
    """Incremental Mean-K append with de-RoPE stage-out during chunked prefill.

    KVMEM, section "Engineering and cost ...": proactive stage-out creates the
    raw-K copy (the reconstruction authority) while chunked prefill runs; the
    index of section "Design and trade-offs ... Mean-K" is the per-block mean
    of that position-free K.  Reading: token t of the workspace sits at
    position pos0 + t; the chunk holds post-RoPE keys of tokens
    t0 .. t0+n-1; their raw K is RoPE removed and rounded to bf16
    (nearest-even) into the stage, and every block the chunk touches is
    re-averaged over the staged raw K of all its tokens so far (a partial block
    averages over the tokens it has, and is redone when the next chunk fills
    it).  So after any sequence of appends the index equals the raw-mode
    build over the stage.

    k_chunk: [L, H_kv, n, D] bf16 bits (or floats); stage: [L, H_kv, cap, D]
    uint16 bf16 bits, rows < t0 already staged.
    Returns (stage_out uint16 bits, first touched block b0, means float64
    [L, H_kv, n_touched, D] for blocks b0 .. b0+n_touched-1).
    """
    k = as_f64(k_chunk)
    L, H_kv, n, D = k.shape
    st = np.array(stage, dtype=np.uint16, copy=True)
    if n == 0:
        return st, t0 // block, np.zeros((L, H_kv, 0, D))
    raw = rope_rotate(k, pos0 + t0 + np.arange(n), theta, inverse=True)
    st[:, :, t0:t0 + n, :] = f64_to_bf16_bits(raw)
    t1 = t0 + n
    b0, b1 = t0 // block, -(-t1 // block)
    staged = bf16_bits_to_f64(st[:, :, b0 * block:t1, :])
    means = np.zeros((L, H_kv, b1 - b0, D))
    for b in range(b0, b1):
        lo, hi = b * block, min(t1, (b + 1) * block)
        means[:, :, b - b0, :] = staged[:, :, lo - b0 * block:hi - b0 * block, :].mean(axis=2)
    return st, b0, means


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
