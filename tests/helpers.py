"""Shared helpers for the GPU parity tests (tensor <-> numpy, tolerances)."""

import numpy as np
import torch

import oracle


def bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (what the oracle consumes)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t):
    """Device tensor -> numpy in the form the oracle takes (bf16 as bits)."""
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.detach().cpu().numpy()


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits; subnormal floor 2^-133)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(int))


def assert_rel(got, want, rtol, what, floor=1e-30):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want) / np.maximum(np.abs(want), floor)
    i = int(np.argmax(err))
    assert err[i] <= rtol, f"{what}: max rel err {err[i]:.3e} at {i} (got {got[i]!r}, want {want[i]!r})"
    return float(err.max())


def assert_within_ulp(got_bits, want, what, ulps=1.0, atol=0.0):
    g = oracle.bf16_bits_to_f64(got_bits)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(g - want)
    bound = ulps * bf16_ulp(want) + atol
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond {ulps} ulp + {atol}; first at "
                             f"{np.unravel_index(i, want.shape)}: got {g.ravel()[i]!r}, want {want.ravel()[i]!r}")
    return float(err.max())


def assert_valid_selection(oracle_scores, keep_idx, forced, c_star, rtol):
    """The kept set is F plus c_star candidates, and no dropped candidate beats a
    kept one by more than rtol (GPU and oracle scores may order near-ties differently)."""
    n = len(oracle_scores)
    keep = np.zeros(n, dtype=bool)
    keep[keep_idx] = True
    assert np.all(np.diff(keep_idx) > 0), "keep_idx not strictly ascending"
    assert keep[forced].all(), "a forced position was dropped"
    cand = ~forced
    n_sel = int((keep & cand).sum())
    assert n_sel == min(c_star, int(cand.sum()))
    if n_sel == 0 or n_sel == cand.sum():
        return
    kept_min = oracle_scores[keep & cand].min()
    dropped_max = oracle_scores[~keep & cand].max()
    assert kept_min >= dropped_max * (1 - rtol), (kept_min, dropped_max)
