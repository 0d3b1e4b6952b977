"""Seeded synthetic inputs in the shapes of the scoring workloads.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no RoPE, no means, no softmax, no selection).  Tests and
the benchmark hand the same tensors to the HIP library and to the oracle.

Recipe
------
* Seeds: numpy ``default_rng([cfg_seed, tensor_id, layer])`` on the host;
  on a GPU, ``torch.Generator`` seeded from the same triple through
  ``numpy.random.SeedSequence``.  Host and device draws differ; whichever
  tensor a run uses is the one both sides consume.
* Values are drawn in float32 from N(0, 1) and rounded to bf16 (nearest-even)
  where the workload is bf16.
* Post-RoPE keys and query rows are drawn directly from N(0, 1): RoPE rotates
  each coordinate pair by an angle, and a rotated pair of independent N(0, 1)
  values is again a pair of independent N(0, 1) values, so the draw has
  exactly the distribution of RoPE applied to N(0, 1) raw vectors.
* The 14B-shaped worst case adds "+2 sigma evidence clusters": contiguous runs
  of 64..1024 positions, non-overlapping, covering 20% of [pi, q_s); every
  coordinate of those keys is shifted by +2.0 before rounding.
* Slot maps are seeded permutations of [0, N); page tables are seeded
  permutations of the pool's pages.
"""

import numpy as np
import torch

# tensor ids for the seed triple
T_K, T_Q, T_V, T_SLOTS, T_EVIDENCE, T_PAGES, T_M, T_SCORE, T_INDEX = range(9)

CONFIGS = {
    # Rule mode, tiny: fp32 K, 3 turns of 32 query rows.
    "rule-tiny": dict(mode="rule", seed=0, L=2, H_q=4, H_kv=2, D=64, N=1024, dtype="f32",
                      turns=3, span=32, lam=0.5, pi=16, q_s=992, q_e=1024, C=256, dead_slot=-1),
    # Rule mode, Qwen3-8B-shaped.
    "rule-8b": dict(mode="rule", seed=1, L=36, H_q=32, H_kv=8, D=128, N=32768, dtype="bf16",
                    turns=8, span=64, lam=0.3, pi=64, q_s=32704, q_e=32768, C=8192, dead_slot=-1),
    # Rule mode, 14B-shaped worst case with evidence clusters.
    "rule-14b": dict(mode="rule", seed=2, L=48, H_q=40, H_kv=8, D=128, N=92160, dtype="bf16",
                     turns=12, span=64, lam=0.3, pi=64, q_s=92096, q_e=92160, C=8192, dead_slot=-1,
                     evidence_frac=0.2),
    # Mean-K, 27B-class GQA, 256K-token workspace.
    "meank-256k": dict(mode="meank", seed=3, L=64, H_q=40, H_kv=8, D=128, N=262144, block=32,
                       Mq=512, n_sink=4, n_recent=64, budget=2048, theta=1e6, pos_base=0),
    # Mean-K, 1M-token workspace; scatter reads a packed staging buffer.
    "meank-1m": dict(mode="meank", seed=4, L=64, H_q=40, H_kv=8, D=128, N=1048576, block=32,
                     Mq=1024, n_sink=4, n_recent=64, budget=4096, theta=1e6, pos_base=0,
                     staging=True),
}


def config(name, **overrides):
    c = dict(CONFIGS[name])
    c.update(overrides)
    c["name"] = name
    return c


def _torch_seed(cfg_seed, tensor_id, layer):
    return int(np.random.SeedSequence([cfg_seed, tensor_id, layer]).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))


def _tdtype(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def normal(shape, cfg_seed, tensor_id, dtype="bf16", device="cpu", scale=1.0, shift_rows=None,
           shift=0.0):
    """N(0, scale^2) tensor of ``shape``, drawn one leading-index slice at a time.

    shift_rows: optional boolean numpy mask over axis -2; those rows get +shift
    on every coordinate before rounding to ``dtype``.
    """
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=_tdtype(dtype), device=device)
    lead = shape[0] if len(shape) > 1 else 1
    sub = shape[1:] if len(shape) > 1 else shape
    if shift_rows is not None:
        mask = torch.from_numpy(np.asarray(shift_rows, dtype=bool)).to(device)
    for i in range(lead):
        if torch.device(device).type == "cpu":
            x = np.random.default_rng([cfg_seed, tensor_id, i]).standard_normal(sub, dtype=np.float32)
            x = torch.from_numpy(x)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(_torch_seed(cfg_seed, tensor_id, i))
            x = torch.randn(sub, generator=g, dtype=torch.float32, device=device)
        if scale != 1.0:
            x.mul_(scale)
        if shift_rows is not None:
            x[..., mask, :] += shift
        if len(shape) > 1:
            out[i].copy_(x)
        else:
            out.copy_(x)
        del x
    return out


def evidence_rows(N, lo, hi, frac, cfg_seed):
    """Boolean [N]: non-overlapping runs of 64..1024 positions covering ~frac of [lo, hi)."""
    r = np.random.default_rng([cfg_seed, T_EVIDENCE, 0])
    mask = np.zeros(N, dtype=bool)
    target = int(frac * (hi - lo))
    covered, tries = 0, 0
    while covered < target and tries < 100000:
        tries += 1
        ln = int(r.integers(64, 1025))
        ln = min(ln, target - covered)
        s = int(r.integers(lo, max(lo + 1, hi - ln)))
        if s + ln > hi or mask[max(lo, s - 1):s + ln + 1].any():
            continue
        mask[s:s + ln] = True
        covered += ln
    return mask


def rule_inputs(c, device="cpu"):
    """K [L,H_kv,N,D], per-turn query spans [L,H_q,span,D], slot map [N] int64."""
    ev = None
    if c.get("evidence_frac"):
        ev = evidence_rows(c["N"], c["pi"], c["q_s"], c["evidence_frac"], c["seed"])
    K = normal((c["L"], c["H_kv"], c["N"], c["D"]), c["seed"], T_K, c["dtype"], device,
               shift_rows=ev, shift=2.0)
    spans = [normal((c["L"], c["H_q"], c["span"], c["D"]), c["seed"], T_Q * 1000 + t, c["dtype"], device)
             for t in range(c["turns"])]
    slots = torch.from_numpy(np.random.default_rng([c["seed"], T_SLOTS, 0]).permutation(c["N"]).astype(np.int64))
    return dict(K=K, spans=spans, slots=slots.to(device), evidence=ev)


def memory_vectors(L, H_q, D, cfg_seed, device="cpu"):
    """Random QueryMemory-shaped fp32 [L, H_q, D] (not normalised) for scorer-only tests."""
    return normal((L, H_q, D), cfg_seed, T_M, "f32", device)


def meank_inputs(c, device="cpu", with_k=True, with_v=False):
    """Raw K (and V) [L,H_kv,N,D] bf16 and queries [L,H_q,Mq,D] bf16."""
    out = {}
    if with_k:
        out["K"] = normal((c["L"], c["H_kv"], c["N"], c["D"]), c["seed"], T_K, "bf16", device)
    if with_v:
        out["V"] = normal((c["L"], c["H_kv"], c["N"], c["D"]), c["seed"], T_V, "bf16", device)
    out["Q"] = normal((c["L"], c["H_q"], c["Mq"], c["D"]), c["seed"], T_Q, "bf16", device)
    return out


def index_like(L, H_kv, nB, D, cfg_seed, device="cpu", scale=0.1767766952966369):
    """A bf16 index-shaped tensor drawn directly (default scale 1/sqrt(32), the spread of a 32-mean)."""
    return normal((L, H_kv, nB, D), cfg_seed, T_INDEX, "bf16", device, scale=scale)


def page_permutation(n_sel, pool_pages, cfg_seed):
    """int32 [n_sel]: distinct destination pages drawn from [0, pool_pages)."""
    r = np.random.default_rng([cfg_seed, T_PAGES, 0])
    return torch.from_numpy(r.permutation(pool_pages)[:n_sel].astype(np.int32))


def scores_with_ties(n, cfg_seed, levels=None):
    """fp32 [n] scores; with ``levels`` they are quantised to that many distinct values (ties)."""
    r = np.random.default_rng([cfg_seed, T_SCORE, 0])
    x = r.standard_normal(n).astype(np.float32)
    if levels:
        x = (np.floor((x + 4.0) * (levels / 8.0)) / levels).astype(np.float32)
    return torch.from_numpy(x)
