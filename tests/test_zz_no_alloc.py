"""The top-k entry point that allocates nothing (kvs_topk_select_noalloc), through the C ABI,
against kvs_topk_select with a caller workspace and against the oracle: bit for bit, over calls in
a row that share the library's static device state -- a larger input, then a smaller one, then the
register path that needs no state, then a larger one again."""

import numpy as np
import pytest
import torch

import oracle
from attention_space_retrieval_amd import kvs, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _outputs(n):
    # filled with values no selection writes, so a missed store shows up
    return (torch.full((n,), 7, dtype=torch.uint8, device=DEV), torch.full((n,), -5, dtype=torch.int32, device=DEV),
            torch.full((1,), -1, dtype=torch.int64, device=DEV))


def _host(keep, idx, nk):
    k = int(nk.item())
    return keep.cpu().numpy(), idx[:k].cpu().numpy(), k


@pytest.mark.parametrize("concentrated", [False, True])
def test_noalloc_equals_workspace_call_over_consecutive_calls(concentrated):
    cases = [(92160, None, (0, 64), (92096, 92160), 8192),      # rule-14b's shape: multi-workgroup
             (40000, 5, (0, 100), (39000, 40000), 7000),         # smaller, with ties: same state reused
             (5000, None, (0, 4), (4936, 5000), 1000),           # one register-resident workgroup
             (65537, 3, (0, 1), (65000, 65537), 30000)]          # larger again, one-position last slice
    for i, (n, levels, f0, f1, C) in enumerate(cases):
        print(f"[noalloc] case {i}: n={n} C={C} concentrated={concentrated}", flush=True)
        score = W.scores_with_ties(n, 300 + i, levels)
        if concentrated:                     # every score within ~1e-3 of the mean, as rule scores are
            score = (1.0 + 1e-3 * score).to(torch.float32)
        score = score.to(DEV)
        got = _outputs(n)
        kvs.kvs_topk_select_noalloc(score, f0, f1, C, *got)
        ref = _outputs(n)
        kvs.kvs_topk_select(score, f0, f1, C, *ref)
        torch.cuda.synchronize()
        g_keep, g_idx, g_nk = _host(*got)
        r_keep, r_idx, r_nk = _host(*ref)
        assert g_nk == r_nk
        np.testing.assert_array_equal(g_keep, r_keep)
        np.testing.assert_array_equal(g_idx, r_idx)
        np.testing.assert_array_equal(got[1][g_nk:].cpu().numpy(), np.full(n - g_nk, -5, np.int32))
        o_keep, o_idx, o_nk = oracle.topk_select(score.cpu().numpy(), f0, f1, C)
        assert g_nk == o_nk
        np.testing.assert_array_equal(g_keep, o_keep.astype(np.uint8))
        np.testing.assert_array_equal(g_idx, o_idx)


def test_noalloc_on_a_side_stream():
    """On a stream of its own (not the default one) the entry point finds that stream's device and its
    copy of the static array; the result equals the workspace call's."""
    n, f0, f1, C = 92160, (0, 64), (92096, 92160), 8192
    score = W.scores_with_ties(n, 320, 6).to(DEV)
    ref = _outputs(n)
    kvs.kvs_topk_select(score, f0, f1, C, *ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = _outputs(n)
    with torch.cuda.stream(side):
        kvs.kvs_topk_select_noalloc(score, f0, f1, C, *got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_keep, g_idx, g_nk = _host(*got)
    r_keep, r_idx, r_nk = _host(*ref)
    assert g_nk == r_nk
    np.testing.assert_array_equal(g_keep, r_keep)
    np.testing.assert_array_equal(g_idx, r_idx)


def test_noalloc_replays_in_a_graph():
    """Captured in a HIP graph (the caller it is for) and replayed on fresh scores written into the
    captured buffer, with eager calls of both entry points between the replays: every replay equals
    the eager selection bit for bit."""
    n, f0, f1, C = 92160, (0, 64), (92096, 92160), 8192
    score = torch.empty(n, dtype=torch.float32, device=DEV)
    got = _outputs(n)
    score.copy_(W.scores_with_ties(n, 330, None).to(DEV))
    side = torch.cuda.Stream()                          # warm up off the capture stream first
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvs.kvs_topk_select_noalloc(score, f0, f1, C, *got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvs.kvs_topk_select_noalloc(score, f0, f1, C, *got)
    torch.cuda.synchronize()
    for rep, (seed, levels) in enumerate(((331, None), (332, 4), (333, 50))):
        print(f"[noalloc] graph replay {rep}", flush=True)
        score.copy_(W.scores_with_ties(n, seed, levels).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        g_keep, g_idx, g_nk = _host(*got)
        ref = _outputs(n)
        kvs.kvs_topk_select(score, f0, f1, C, *ref)
        eager = _outputs(n)
        kvs.kvs_topk_select_noalloc(score, f0, f1, C, *eager)
        torch.cuda.synchronize()
        for keep, idx, nk in (_host(*ref), _host(*eager)):
            assert g_nk == nk
            np.testing.assert_array_equal(g_keep, keep)
            np.testing.assert_array_equal(g_idx, idx)
