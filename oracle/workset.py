"""Differential working-set update of the execution view (test infrastructure only).

KVMEM, section "Engineering and cost: tiered movement, page-table aliasing and
position-consistent reconstruction": consecutive steps' working sets overlap,
and only blocks that the step selects but the GPU page pool no longer holds
(W_t minus G_{t-1}) are materialised again; the page distinguishes retained,
incoming and outgoing blocks.  The page table maps physical pages to the
compact logical order, and RoPE must match a block's new compact position.

Readings (the difference equation itself was lost in extraction):

* W_t (this step's selection) and G_{t-1} (the blocks resident after the
  previous step) are ascending block ids; a block's compact index is its rank
  in that list, so block r of the view sits at positions pos_base + 32 r ... +31.
* retained = W_t and G_{t-1}: the block keeps its physical page.  If its
  compact index moved, its K is rebuilt from raw K (the page's reconstruction
  authority) at the new positions pos_base + 32 r ... +31, exactly as the
  re-RoPE scatter writes it; V carries no position and is untouched.  (Rotating
  the pool's bf16 copy by the position delta instead would round once more per
  move, so a block that moves over many steps would drift away from raw K.)
  pos_base is the same in consecutive steps: a retained block whose compact
  index did not move is left as it is.
* incoming = W_t minus G_{t-1}: takes a free page (a page no retained block
  holds), the free pages handed out in ascending page order to the incoming
  blocks in ascending compact order, and is written like the re-RoPE scatter:
  raw K rotated to its compact positions, V copied.
* outgoing = G_{t-1} minus W_t: its page is released (contents left as they are).
"""

import numpy as np

from .bf16 import as_f64
from .rope import rope_rotate


def working_set_diff(prev_blocks, prev_pages, new_blocks, pool_pages):
    """Classes and the new page table.

    Returns (pages [n_new] int64, old_rank [n_new] int64 (-1 = incoming),
    outgoing_pages [n_out] int64 in G_{t-1} order).
    """
    prev_blocks = [int(b) for b in prev_blocks]
    prev_pages = [int(p) for p in prev_pages]
    new_blocks = [int(b) for b in new_blocks]
    rank = {b: i for i, b in enumerate(prev_blocks)}
    old_rank = np.array([rank.get(b, -1) for b in new_blocks], dtype=np.int64)
    held = {prev_pages[i] for i in old_rank if i >= 0}
    free = [p for p in range(pool_pages) if p not in held]
    pages = np.empty(len(new_blocks), dtype=np.int64)
    k = 0
    for r, i in enumerate(old_rank):
        if i >= 0:
            pages[r] = prev_pages[i]
        else:
            pages[r] = free[k]
            k += 1
    kept = set(new_blocks)
    outgoing = np.array([p for b, p in zip(prev_blocks, prev_pages) if b not in kept], dtype=np.int64)
    return pages, old_rank, outgoing


def working_set_update(k_src, v_src, prev_blocks, prev_pages, new_blocks, pos_base, theta,
                       k_pool, v_pool, block=32):
    """Apply the update to the pools.

    k_src, v_src: [L, H_kv, src_tokens, D] raw (position-free) K and V;
    k_pool, v_pool: [L, H_kv, pool_pages*block, D] current pool contents.
    Returns (k_pool_out float64, v_pool_out (v_pool's dtype), pages, old_rank, outgoing_pages).
    """
    pool_pages = k_pool.shape[2] // block
    pages, old_rank, outgoing = working_set_diff(prev_blocks, prev_pages, new_blocks, pool_pages)
    k_out = as_f64(k_pool).copy()
    v_out = np.array(v_pool, copy=True)
    for r, b in enumerate(new_blocks):
        rows = slice(int(pages[r]) * block, (int(pages[r]) + 1) * block)
        if old_rank[r] == r:
            continue                                  # retained at the same compact index
        src = slice(int(b) * block, (int(b) + 1) * block)
        pos = pos_base + block * r + np.arange(block)
        k_out[:, :, rows, :] = rope_rotate(as_f64(k_src[:, :, src, :]), pos, theta)
        if old_rank[r] < 0:                           # incoming: V copied; a moved block's V stays
            v_out[:, :, rows, :] = v_src[:, :, src, :]
    return k_out, v_out, pages, old_rank, outgoing
