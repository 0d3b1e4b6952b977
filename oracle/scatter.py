"""Re-RoPE scatter into the execution view (test infrastructure only).

KVMEM, section "Engineering and cost: tiered movement, page-table aliasing and
position-consistent reconstruction": the execution view maps non-contiguous
physical pages to a compact logical order through a page table; raw
(position-free) K is the reconstruction authority and RoPE is re-applied at
the new compact position, while V carries no position and is copied as is.
The packed-and-pipelined path ends with a GPU scatter + re-RoPE.

Reading: selected block r (ascending original order) is logical block r of
the view, occupies positions pos_base + block*r ... + block-1, and lands on
physical page page_table[r] (identity when None).
"""

import numpy as np

from .bf16 import as_f64
from .rope import rope_rotate


def rerope_scatter(k_src, v_src, src_block, page_table, pos_base, theta,
                   k_pool, v_pool, block=32):
    """Return (k_pool_out float64, v_pool_out same dtype as v_pool).

    k_src, v_src: [L, H_kv, src_tokens, D]; src_block: [n_sel] block ids into
    the source; page_table: [n_sel] destination pages or None;
    k_pool, v_pool: [L, H_kv, pool_pages*block, D] initial pool contents
    (pages that receive no block keep them).
    """
    k_out = as_f64(k_pool).copy()
    v_out = np.array(v_pool, copy=True)
    n_sel = len(src_block)
    dst = np.arange(n_sel) if page_table is None else np.asarray(page_table)
    for r in range(n_sel):
        b, p = int(src_block[r]), int(dst[r])
        src = slice(b * block, (b + 1) * block)
        out = slice(p * block, (p + 1) * block)
        pos = pos_base + block * r + np.arange(block)
        k_out[:, :, out, :] = rope_rotate(as_f64(k_src[:, :, src, :]), pos, theta)
        v_out[:, :, out, :] = v_src[:, :, src, :]
    return k_out, v_out
