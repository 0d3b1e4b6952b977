"""Slow, plain float64 CPU oracle for attention-space KV scoring and budgeted top-k.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code, constant table or helper with
the HIP library; the two meet only through the seeded input generators, which
hold none of the method's arithmetic.

Sources (cited by page title and section/equation in every function):

* IntentKV -- "Cross-turn intent-aware KV cache pruning for multi-turn
  reasoning agents" (Chinese rendering of arXiv 2606.09916): Sec. 3.1 Eq. (1)
  budgeted top-k with a forced set, Sec. 3.2 Eq. (2) QueryMemory,
  Eqs. (3)-(4) rule score, abstract/Sec. 1 slot-map redirect to a dead slot.
* KVMEM -- "Virtualising million-token agent workspaces onto a laptop GPU":
  section "Design and trade-offs: step-level attention trigger and Mean-K
  model-native retrieval" (Mean-K index and block relevance R_b; both display
  equations were lost in extraction, only their symbol glossaries remain) and
  section "Engineering and cost: tiered movement, page-table aliasing and
  position-consistent reconstruction" (execution view, re-RoPE from raw K,
  differential working-set update, proactive stage-out).

Every function is the plain definition in float64.  bf16 inputs are widened
from their uint16 bit patterns, which is exact.

Parity status: every function here is pinned by the CPU tests against closed
forms, invariants, library special cases and brute force, except for the
conventions no page value can confirm (listed as "parity unpinned" in the
function docstrings): the decay value lambda the IntentKV paper used, the RoPE
pairing of the pages' models, which layer-heads KVMEM lets vote, how positions
on the dead slot enter later rule scoring, and the window score beyond its
plainest reading (sum of per-row softmaxes, no pooling).
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, as_f64
from .qmem import qmem_update, enc_span
from .rule import forced_mask, rule_score, rule_score_paged, window_score
from .select import topk_select, slotmap_redirect, meank_select
from .rope import rope_omega, rope_rotate
from .meank import meank_build, meank_append, meank_score, candidate_blocks
from .scatter import rerope_scatter
from .workset import working_set_diff, working_set_update

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "as_f64",
    "qmem_update", "enc_span",
    "forced_mask", "rule_score", "rule_score_paged", "window_score",
    "topk_select", "slotmap_redirect", "meank_select",
    "rope_omega", "rope_rotate",
    "meank_build", "meank_append", "meank_score", "candidate_blocks",
    "rerope_scatter",
    "working_set_diff", "working_set_update",
]
