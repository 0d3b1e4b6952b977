"""The hot path inside a HIP graph, and on concurrent streams.

A rule turn (QueryMemory update, rule score, top-k, slot redirect) and a Mean-K
step (index build, block relevance, top-k, re-RoPE scatter) are captured once
with every output and workspace preallocated, then replayed several times on
fresh inputs written into the captured buffers, with eager work and
synchronisations between the replays.  Every replay must equal the eager
calls on the same inputs bit for bit: the library launches only kernels (no
memset, copy, allocation or synchronisation) and every kernel is
deterministic.  The rule cache is longer than 32768 positions, so the
multi-workgroup top-k and its workspace are part of the graph.
"""

import pytest
import torch

from attention_space_retrieval_amd import kvs, workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class Turn:
    """Preallocated buffers for one rule turn and one Mean-K step."""

    def __init__(self):
        # rule mode
        self.L, self.H_q, self.H_kv, self.D, self.N = 2, 8, 2, 128, 40000
        self.pi, self.q_s, self.q_e, self.C, self.lam = 16, 39936, 40000, 4096, 0.3
        L, H_q, H_kv, D, N = self.L, self.H_q, self.H_kv, self.D, self.N
        self.K = torch.empty((L, H_kv, N, D), dtype=torch.bfloat16, device=DEV)
        self.span = torch.empty((L, H_q, 64, D), dtype=torch.bfloat16, device=DEV)
        self.M = torch.empty((L, H_q, D), dtype=torch.float32, device=DEV)
        self.slots = torch.empty(N, dtype=torch.int64, device=DEV)
        self.rule = torch.empty(N, dtype=torch.float32, device=DEV)
        self.ws_rule = torch.empty(kvs.kvs_rule_score_workspace(L, H_q, H_kv, N), dtype=torch.uint8, device=DEV)
        self.keep = torch.empty(N, dtype=torch.uint8, device=DEV)
        self.idx = torch.empty(N, dtype=torch.int32, device=DEV)
        self.nk = torch.empty(1, dtype=torch.int64, device=DEV)
        need = kvs.kvs_topk_workspace(N)
        assert need > 0, "the rule cache should take the multi-workgroup top-k"
        self.ws_topk = torch.empty(need, dtype=torch.uint8, device=DEV)
        self.slots_out = torch.empty(N, dtype=torch.int64, device=DEV)
        # Mean-K mode
        self.mL, self.mHq, self.mHkv, self.mN, self.Mq = 2, 8, 2, 32 * 300, 40
        self.sink, self.recent, self.budget, self.theta = 4, 8, 64, 1e6
        mL, mHq, mHkv, mN, Mq = self.mL, self.mHq, self.mHkv, self.mN, self.Mq
        self.nB = mN // 32
        self.Kraw = torch.empty((mL, mHkv, mN, D), dtype=torch.bfloat16, device=DEV)
        self.V = torch.empty_like(self.Kraw)
        self.Q = torch.empty((mL, mHq, Mq, D), dtype=torch.bfloat16, device=DEV)
        self.index = torch.empty((mL, mHkv, self.nB, D), dtype=torch.bfloat16, device=DEV)
        self.R = torch.empty(self.nB, dtype=torch.float32, device=DEV)
        self.ws_mk = torch.empty(kvs.kvs_meank_score_workspace(mL, mHq, mHkv, Mq, self.nB), dtype=torch.uint8,
                                 device=DEV)
        self.keep_m = torch.empty(self.nB, dtype=torch.uint8, device=DEV)
        self.idx_m = torch.empty(self.nB, dtype=torch.int32, device=DEV)
        self.nk_m = torch.empty(1, dtype=torch.int64, device=DEV)
        self.k_pool = torch.empty((mL, mHkv, 32 * self.budget, D), dtype=torch.bfloat16, device=DEV)
        self.v_pool = torch.empty_like(self.k_pool)
        self.err = torch.empty(1, dtype=torch.int32, device=DEV)

    def fill(self, seed):
        """Fresh inputs written into the same buffers (the captured addresses)."""
        self.K.copy_(W.normal(tuple(self.K.shape), seed, W.T_K, "bf16", DEV))
        self.span.copy_(W.normal(tuple(self.span.shape), seed, W.T_Q, "bf16", DEV))
        self.M.copy_(W.memory_vectors(self.L, self.H_q, self.D, seed, DEV))
        g = torch.Generator(device="cpu").manual_seed(seed)
        self.slots.copy_(torch.randperm(self.N + 100, generator=g)[: self.N].to(DEV))
        self.Kraw.copy_(W.normal(tuple(self.Kraw.shape), seed, W.T_K + 1, "bf16", DEV))
        self.V.copy_(W.normal(tuple(self.V.shape), seed, W.T_V, "bf16", DEV))
        self.Q.copy_(W.normal(tuple(self.Q.shape), seed, W.T_Q + 1, "bf16", DEV))
        for t in (self.k_pool, self.v_pool):
            t.fill_(0)
        self.err.zero_()

    def calls(self):
        self.rule_calls()
        self.meank_calls()

    def rule_calls(self):
        kvs.kvs_qmem_update(self.span, self.lam, self.M, False)
        kvs.kvs_rule_score(self.K, self.M, self.pi, self.q_s, self.q_e, rule=self.rule, ws=self.ws_rule)
        kvs.kvs_topk_select(self.rule, (0, self.pi), (self.q_s, self.q_e), self.C, self.keep, self.idx, self.nk,
                            ws=self.ws_topk)
        kvs.kvs_slotmap_redirect(self.slots, self.keep, -1, self.slots_out)

    def meank_calls(self):
        kvs.kvs_meank_build(self.Kraw, index=self.index)
        kvs.kvs_meank_score(self.Q, self.index, self.sink, self.recent, R=self.R, ws=self.ws_mk)
        kvs.kvs_topk_select(self.R, (0, self.sink), (self.nB - self.recent, self.nB), self.budget, self.keep_m,
                            self.idx_m, self.nk_m)
        kvs.kvs_rerope_scatter(self.Kraw, self.V, self.idx_m[: self.budget], None, self.budget, 0, self.theta,
                               self.k_pool, self.v_pool, self.err)

    def outputs(self):
        return {name: getattr(self, name).clone() for name in
                ("M", "rule", "keep", "idx", "nk", "slots_out", "index", "R", "keep_m", "idx_m", "nk_m",
                 "k_pool", "v_pool", "err")}


def test_rule_turn_and_meank_step_replay_in_a_graph():
    t = Turn()
    # capture (torch warms the calls up on a side stream first, as its graph API asks)
    t.fill(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        t.calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        t.calls()
    torch.cuda.synchronize()
    for rep, seed in enumerate((101, 102, 103)):
        print(f"[graph] replay {rep} on inputs of seed {seed}", flush=True)
        t.fill(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = t.outputs()
        t.fill(seed)                     # eager work between the replays: the same inputs, the plain calls
        t.calls()
        torch.cuda.synchronize()
        want = t.outputs()
        assert int(want["nk"].item()) == t.C and int(want["nk_m"].item()) == t.budget
        assert int(want["err"].item()) == 0
        for name in want:
            assert torch.equal(got[name], want[name]), f"replay {rep}: {name} differs from the eager calls"


def test_rule_turn_and_meank_step_on_concurrent_streams():
    """The two modes on two streams at once give what they give one after the other."""
    t = Turn()
    t.fill(200)
    torch.cuda.synchronize()
    t.calls()
    torch.cuda.synchronize()
    want = t.outputs()
    t.fill(200)
    a, b = torch.cuda.Stream(), torch.cuda.Stream()
    a.wait_stream(torch.cuda.current_stream())
    b.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(a):
        t.rule_calls()
    with torch.cuda.stream(b):
        t.meank_calls()
    torch.cuda.current_stream().wait_stream(a)
    torch.cuda.current_stream().wait_stream(b)
    torch.cuda.synchronize()
    got = t.outputs()
    for name in want:
        assert torch.equal(got[name], want[name]), f"{name} differs between concurrent and sequential calls"


def test_rule_scores_on_concurrent_streams_share_the_device():
    """Two rule scores with their own workspaces, on two streams at once, next to a Mean-K score
    on a third: each equals its call alone, bit for bit.  The rule score's persistent workgroups
    claim chunks from queues in their own workspace and never rely on how many of them are
    resident, so sharing the CUs with other kernels changes only the timing."""
    shapes = [(2, 32, 8, 128, 131073), (3, 40, 8, 128, 50000)]     # G = 4 and G = 5
    jobs = []
    for i, (L, H_q, H_kv, D, N) in enumerate(shapes):
        K = W.normal((L, H_kv, N, D), 300 + i, W.T_K, "bf16", DEV)
        M = W.memory_vectors(L, H_q, D, 300 + i, DEV)
        ws = torch.empty(kvs.kvs_rule_score_workspace(L, H_q, H_kv, N), dtype=torch.uint8, device=DEV)
        out = torch.empty(N, dtype=torch.float32, device=DEV)
        jobs.append((K, M, ws, out, N))
    mk_Q = W.normal((4, 32, 512, 128), 310, W.T_Q, "bf16", DEV)
    mk_index = W.normal((4, 8, 8192, 128), 310, W.T_K, "bf16", DEV)
    mk_R = torch.empty(8192, dtype=torch.float32, device=DEV)
    mk_ws = torch.empty(kvs.kvs_meank_score_workspace(4, 32, 8, 512, 8192), dtype=torch.uint8, device=DEV)
    alone = []
    for K, M, ws, out, N in jobs:
        kvs.kvs_rule_score(K, M, 5, N - 64, N, rule=out, ws=ws)
        torch.cuda.synchronize()
        alone.append(out.clone())
    kvs.kvs_meank_score(mk_Q, mk_index, 4, 64, R=mk_R, ws=mk_ws)
    torch.cuda.synchronize()
    mk_alone = mk_R.clone()
    for rep in range(3):
        for _, _, _, out, _ in jobs:
            out.fill_(float("nan"))
        streams = [torch.cuda.Stream() for _ in range(3)]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(streams[2]):
            kvs.kvs_meank_score(mk_Q, mk_index, 4, 64, R=mk_R, ws=mk_ws)
        for s, (K, M, ws, out, N) in zip(streams[:2], jobs):
            with torch.cuda.stream(s):
                kvs.kvs_rule_score(K, M, 5, N - 64, N, rule=out, ws=ws)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for (_, _, _, out, _), want in zip(jobs, alone):
            assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"round {rep}"
        assert torch.equal(mk_R.view(torch.int32), mk_alone.view(torch.int32))
