"""Benchmark: one step = the whole hot path on one GPU, inputs resident in HBM.

A step is an IntentKV turn on the rule-mode cache (QueryMemory update, rule
score, top-k with the forced set, slot redirect) followed by a KVMEM agent step
on the Mean-K workspace (index build from raw K, block scoring, sink/recent +
budget selection, re-RoPE scatter of the selected K/V blocks into the pool).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload rule-14b+meank-1m]

The default workload is the largest that fits one GPU: the 14B-shaped rule
cache (N = 92160, IntentKV's worst case) and the 1M-token Mean-K workspace
(32768 blocks, budget 4096, scatter from a packed staging buffer through a page
table).  rule-8b+meank-256k is the smaller pair.

Prints one JSON line.  `value` counts K-cache tokens scored per second over the
whole step (the rule cache's N plus the Mean-K workspace's N).  Per-call times
come from HIP events on the stream the library launches on; `roofline` is the
call with the largest share of the step, priced against MI355X's published
peaks; `next_rows` times the calls beyond the step (paged rule score, window
score, Mean-K append, working-set update) on the same workload's shapes after
the timed steps, outside `value`.  `traffic` (per call) is the HBM bytes per launch that
rocprofv3's FETCH_SIZE/WRITE_SIZE counters measured, read from the committed
summary under profiles/ and scaled by the counters' reading of a device copy of
known size, or null when the kernel source has changed since.  `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload and scales
it linearly to a whole step.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_space_retrieval_amd import kvs, workloads as W  # noqa: E402

METRIC = "K-cache tokens scored/s + HBM GB/s (rule+top-k); Mean-K scoring TFLOP/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# Sustained rate of R_b's instruction mix (bf16 MFMA 32x32x16 with one fma + exp2 + add per logit
# interleaved) in a register-only loop over all 256 CUs at 4-16 waves per SIMD: 1.51-1.57 PFLOP/s,
# against ~1.96 PFLOP/s for the MFMAs alone (the clock does not hold 2.4 GHz under either load).
MIX_CEILING_TFLOPS = 1570.0
# The same mix at the engine's two waves per SIMD with random bf16 operands (N(0, 1/4)) in the
# registers instead of constant ones: the switching of the operand bits holds the chip at its power
# cap, and the loop runs at 1.28-1.30 PFLOP/s (1.63 on zero operands, 1.70 without the exp2).
MIX_CEILING_RANDOM_TFLOPS = 1290.0
WORKLOADS = {"rule-8b+meank-256k": ("rule-8b", "meank-256k"),
             "rule-14b+meank-1m": ("rule-14b", "meank-1m")}
# kernels each call launches (rocprofv3 short names); a tuple lists alternatives of which the
# call launches one, chosen by the sizes (the window score's first pass runs two-wave workgroups
# for windows of at most 128 rows per KV group; its second pass always does); "name*k" is a kernel
# the call launches k times.  Top-k runs one register-resident workgroup up to 8192 or 32768
# scores and the multi-workgroup path above that (rule-14b's 92160).
TOPK_MW = ["topk_mw_init", "topk_mw_minmax", "topk_mw_pass*4", "topk_mw_count", "topk_mw_emit"]
CALL_KERNELS = {
    "kvs_qmem_update": ["qmem_kernel<128, true>"],
    # bf16 keys, G <= 8: the work-queue fold; the last template argument is the workgroups per CU
    # its LDS allows (3 at G = 4, 2 at G = 5), the third the chunk length
    "kvs_rule_score": ["rule_fold_reset", "rule_fold_queue<128, false, 1024, 3>", "rule_fold_colsum<4>"],
    # the redirect runs inside the multi-workgroup emit, and as its own kernel after a one-workgroup
    # selection
    "kvs_topk_select_redirect[rule]": ["topk_wg_kernel<8>", "slotmap_kernel"],
    "kvs_topk_select[meank]": ["topk_wg_kernel<2>"],
    "kvs_meank_build": ["meank_build_raw<128>"],
    "kvs_meank_score": ["meank_pass_dma<true>", "meank_pass_dma<false>", "meank_reduce<false>"],
    "kvs_rerope_scatter": ["rerope_scatter_kernel<128>", "v_scatter_kernel<128>"],
    # rows beyond the step (timed after it): the paged rule score takes 768-position chunks
    "kvs_rule_score_paged": ["rule_fold_reset", "rule_fold_queue<128, true, 768, 3>", "rule_fold_colsum<4>"],
    "kvs_window_score": [("meank_pass<true, true, 2, 128>", "meank_pass<true, true, 4, 128>"), "meank_lse_merge",
                         "meank_pass<false, true, 2, 128>",
                         "meank_reduce<true>"],
    "kvs_meank_append": ["meank_append_kernel<128>"],
    "kvs_working_set_update": ["workset_diff", "workset_apply<128, true>"],
}


def call_kernels(workload):
    """CALL_KERNELS with the top-k kernels the workload's sizes select."""
    ck = dict(CALL_KERNELS)
    if workload == "rule-14b+meank-1m":
        ck["kvs_rule_score"] = ["rule_fold_reset", "rule_fold_queue<128, false, 1024, 2>", "rule_fold_colsum<4>"]
        ck["kvs_topk_select_redirect[rule]"] = TOPK_MW              # n = 92160
        ck["kvs_topk_select[meank]"] = ["topk_wg_kernel<8>"]       # n = 32768 blocks
        # the 1M workspace keeps no V beside raw K (the scatter reads the packed staging buffers), so
        # the working-set update there moves K only
        ck["kvs_working_set_update"] = ["workset_diff", "workset_apply<128, false>"]
    return ck


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Setup:
    """Device-resident inputs, outputs and workspaces for one step."""

    def __init__(self, rule_name, meank_name, dev):
        self.dev = dev
        c = self.rc = W.config(rule_name)
        inp = W.rule_inputs(c, dev)
        self.K = inp["K"]
        self.spans = inp["spans"]
        self.slots = inp["slots"]
        self.M = torch.empty((c["L"], c["H_q"], c["D"]), dtype=torch.float32, device=dev)
        for t, q in enumerate(self.spans[:-1]):          # earlier turns build the session state
            kvs.kvs_qmem_update(q, c["lam"], self.M, t == 0)
        self.rule = torch.empty(c["N"], dtype=torch.float32, device=dev)
        self.ws_rule = torch.empty(kvs.kvs_rule_score_workspace(c["L"], c["H_q"], c["H_kv"], c["N"]),
                                   dtype=torch.uint8, device=dev)
        self.keep_r = torch.empty(c["N"], dtype=torch.uint8, device=dev)
        self.ws_topk_r = torch.empty(max(1, kvs.kvs_topk_workspace(c["N"])), dtype=torch.uint8, device=dev)
        self.idx_r = torch.empty(c["N"], dtype=torch.int32, device=dev)
        self.nk_r = torch.empty(1, dtype=torch.int64, device=dev)
        self.slots_out = torch.empty_like(self.slots)

        m = self.mc = W.config(meank_name)
        self.nB = m["N"] // 32
        mi = W.meank_inputs(m, dev, with_k=True, with_v=not m.get("staging"))
        self.Kraw, self.Q = mi["K"], mi["Q"]
        self.n_sel = min(m["budget"], self.nB)
        if m.get("staging"):
            # packed staging buffers stand in for the host->device batch of selected blocks
            shp = (m["L"], m["H_kv"], 32 * self.n_sel, m["D"])
            self.k_src = W.normal(shp, m["seed"], W.T_K + 10, "bf16", dev)
            self.v_src = W.normal(shp, m["seed"], W.T_V + 10, "bf16", dev)
            self.src_block = torch.arange(self.n_sel, dtype=torch.int32, device=dev)
            self.page_table = W.page_permutation(self.n_sel, self.n_sel, m["seed"]).to(dev)
        else:
            self.k_src, self.v_src = self.Kraw, mi["V"]
            self.src_block = None                        # the selection itself
            self.page_table = None
        self.index = torch.empty((m["L"], m["H_kv"], self.nB, m["D"]), dtype=torch.bfloat16, device=dev)
        self.R = torch.empty(self.nB, dtype=torch.float32, device=dev)
        self.ws_mk = torch.empty(kvs.kvs_meank_score_workspace(m["L"], m["H_q"], m["H_kv"], m["Mq"], self.nB),
                                 dtype=torch.uint8, device=dev)
        self.keep_m = torch.empty(self.nB, dtype=torch.uint8, device=dev)
        self.ws_topk_m = torch.empty(max(1, kvs.kvs_topk_workspace(self.nB)), dtype=torch.uint8, device=dev)
        self.idx_m = torch.empty(self.nB, dtype=torch.int32, device=dev)
        self.nk_m = torch.empty(1, dtype=torch.int64, device=dev)
        pool = (m["L"], m["H_kv"], 32 * self.n_sel, m["D"])
        self.k_pool = torch.empty(pool, dtype=torch.bfloat16, device=dev)
        self.v_pool = torch.empty(pool, dtype=torch.bfloat16, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    # (name, callable) in step order
    def calls(self):
        c, m = self.rc, self.mc
        nB = self.nB
        src = self.src_block if self.src_block is not None else self.idx_m[: self.n_sel]
        return [
            ("kvs_qmem_update", lambda: kvs.kvs_qmem_update(self.spans[-1], c["lam"], self.M, False)),
            ("kvs_rule_score", lambda: kvs.kvs_rule_score(self.K, self.M, c["pi"], c["q_s"], c["q_e"],
                                                          rule=self.rule, ws=self.ws_rule)),
            ("kvs_topk_select_redirect[rule]", lambda: kvs.kvs_topk_select_redirect(
                self.rule, (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"], self.slots, c["dead_slot"], self.keep_r,
                self.idx_r, self.nk_r, self.slots_out, ws=self.ws_topk_r)),
            ("kvs_meank_build", lambda: kvs.kvs_meank_build(self.Kraw, index=self.index)),
            ("kvs_meank_score", lambda: kvs.kvs_meank_score(self.Q, self.index, m["n_sink"], m["n_recent"],
                                                            R=self.R, ws=self.ws_mk)),
            ("kvs_topk_select[meank]", lambda: kvs.kvs_topk_select(
                self.R, (0, m["n_sink"]), (nB - m["n_recent"], nB), m["budget"], self.keep_m, self.idx_m,
                self.nk_m, ws=self.ws_topk_m)),
            ("kvs_rerope_scatter", lambda: kvs.kvs_rerope_scatter(
                self.k_src, self.v_src, src, self.page_table, self.n_sel, m["pos_base"], m["theta"],
                self.k_pool, self.v_pool, self.err)),
        ]

    def work(self):
        """Algorithmic bytes or flops of each call (what the method must move or compute)."""
        c, m = self.rc, self.mc
        N, nB = c["N"], self.nB
        LG_r = c["L"] * c["H_kv"]
        blk = m["L"] * m["H_kv"] * 32 * m["D"] * 2           # bytes of one 32-token block over all heads
        cand = nB - m["n_sink"] - m["n_recent"]
        return {
            "kvs_qmem_update": ("hbm", c["L"] * c["H_q"] * c["span"] * c["D"] * 2 + 2 * c["L"] * c["H_q"] * c["D"] * 4),
            "kvs_rule_score": ("hbm", LG_r * N * c["D"] * 2 + c["L"] * c["H_q"] * c["D"] * 4 + 4 * N),
            "kvs_topk_select_redirect[rule]": ("hbm", 4 * N + N + 4 * c["C"] + 16 * N),
            "kvs_meank_build": ("hbm", m["L"] * m["H_kv"] * m["N"] * m["D"] * 2 + m["L"] * m["H_kv"] * nB * m["D"] * 2),
            "kvs_meank_score": ("mfma", 2.0 * m["Mq"] * m["H_q"] * m["L"] * cand * m["D"]),
            "kvs_topk_select[meank]": ("hbm", 4 * nB + nB + 4 * m["budget"]),
            "kvs_rerope_scatter": ("hbm", 4 * self.n_sel * blk),
        }


class NextRows:
    """Inputs for the rows beyond the step, at the same workload's shapes.

    * kvs_rule_score_paged: the rule cache read through a permuted slot map from a
      token-major pool with 4096 spare slots.
    * kvs_window_score: the rule cache with a 32-row window of query rows per head.
    * kvs_meank_append: an 8192-token chunk of the Mean-K workspace appended after
      an 8192-token prefix (stage-out and index of the touched blocks).
    * kvs_working_set_update: the step's selection against a previous one that
      shares half of its blocks, on the step's page pool.
    """

    def __init__(self, s, dev):
        c, m = s.rc, s.mc
        self.s = s
        L, H_q, H_kv, D, N = c["L"], c["H_q"], c["H_kv"], c["D"], c["N"]
        r = np.random.default_rng([c["seed"], 99])
        perm = torch.from_numpy(r.permutation(N + 4096)[:N].copy()).to(dev)
        self.pool = torch.empty((L, N + 4096, H_kv, D), dtype=torch.bfloat16, device=dev)
        self.pool[:, perm] = s.K.permute(0, 2, 1, 3)
        self.slots = perm
        self.rule_p = torch.empty_like(s.rule)
        self.W = 32
        self.Qw = W.normal((L, H_q, self.W, D), c["seed"], W.T_Q + 40, "bf16", dev)
        self.win = torch.empty_like(s.rule)
        self.ws_win = torch.empty(kvs.kvs_window_score_workspace(L, H_q, H_kv, self.W, N), dtype=torch.uint8,
                                  device=dev)
        Lm, Hm, Dm = m["L"], m["H_kv"], m["D"]
        self.n_app, self.t0 = 8192, 8192
        cap = self.t0 + self.n_app
        self.chunk = s.Kraw[:, :, self.t0:cap].contiguous()
        self.stage = torch.zeros((Lm, Hm, cap, Dm), dtype=torch.bfloat16, device=dev)
        self.app_index = torch.zeros((Lm, Hm, cap // 32, Dm), dtype=torch.bfloat16, device=dev)
        kvs.kvs_meank_append(s.Kraw[:, :, :self.t0].contiguous(), 0, self.stage, self.app_index)
        nB, budget = s.nB, s.n_sel
        new = np.sort(r.choice(nB, budget, replace=False))
        keep = new[np.sort(r.choice(budget, budget // 2, replace=False))]
        others = np.setdiff1d(np.arange(nB), new)
        prev = np.sort(np.concatenate([keep, r.choice(others, budget - len(keep), replace=False)]))
        prev_pages = r.permutation(budget)
        rank = {int(b): i for i, b in enumerate(prev)}
        self.n_moved = sum(1 for i, b in enumerate(new) if int(b) in rank and rank[int(b)] != i)
        self.n_incoming = sum(1 for b in new if int(b) not in rank)
        i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device=dev)
        self.prev, self.prev_pages, self.new = i32(prev), i32(prev_pages), i32(new)
        self.ws_ws = torch.empty(kvs.kvs_working_set_workspace(budget), dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def calls(self):
        s, c, m = self.s, self.s.rc, self.s.mc
        return [
            ("kvs_rule_score_paged", lambda: kvs.kvs_rule_score_paged(
                self.pool, self.slots, s.M, c["pi"], c["q_s"], c["q_e"], rule=self.rule_p, ws=s.ws_rule)),
            ("kvs_window_score", lambda: kvs.kvs_window_score(
                s.K, self.Qw, c["pi"], c["q_s"], c["q_e"], score=self.win, ws=self.ws_win)),
            ("kvs_meank_append", lambda: kvs.kvs_meank_append(self.chunk, self.t0, self.stage, self.app_index)),
            ("kvs_working_set_update", lambda: kvs.kvs_working_set_update(
                s.Kraw, s.v_src if s.src_block is None else None, self.prev, self.prev_pages, self.new,
                m["pos_base"], m["theta"], s.k_pool, s.v_pool if s.src_block is None else None,
                err_flag=self.err, ws=self.ws_ws)),
        ]

    def work(self):
        s, c, m = self.s, self.s.rc, self.s.mc
        N, LG_r = c["N"], c["L"] * c["H_kv"]
        kbytes = LG_r * N * c["D"] * 2
        blk = m["L"] * m["H_kv"] * 32 * m["D"] * 2
        n_blk = -(-(self.t0 + self.n_app) // 32) - self.t0 // 32
        v_too = 2 if s.src_block is None else 1
        return {
            "kvs_rule_score_paged": ("hbm", kbytes + 8 * N + c["L"] * c["H_q"] * c["D"] * 4 + 4 * N),
            "kvs_window_score": ("hbm", kbytes + c["L"] * c["H_q"] * self.W * c["D"] * 2 + 4 * N),
            "kvs_meank_append": ("hbm", 2 * m["L"] * m["H_kv"] * self.n_app * m["D"] * 2
                                 + m["L"] * m["H_kv"] * n_blk * m["D"] * 2),
            "kvs_working_set_update": ("hbm", 2 * self.n_moved * blk + 2 * v_too * self.n_incoming * blk),
        }


def measured_traffic(workload):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary.

    A call's figure is null when the summary is missing or when the source of
    any of its kernels has changed since the counters were taken."""
    from attention_space_retrieval_amd import rocprof_summary as rs
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_all-kernels_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        summ = json.load(f)["kernels"]
    out = {}
    for call, kernels in call_kernels(workload).items():
        total = 0.0
        for k in kernels:
            alts = k if isinstance(k, tuple) else (k,)   # alternatives share one source file
            times = 1
            if len(alts) == 1 and "*" in alts[0]:
                name, n = alts[0].rsplit("*", 1)
                alts, times = (name,), int(n)
            e = next((summ[n] for n in alts if n in summ), None)
            if e is None or e["source_sha256"] != rs.source_hash(rs.base_name(alts[0])):
                total = None
                break
            total += times * (e["read_bytes_mean"] + e["write_bytes_mean"])
        out[call] = total
    return out


def run_calls(calls, steps, warmup):
    """Warm up, then time `steps` passes over `calls` with HIP events between the calls."""
    for _ in range(warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for i, (_, f) in enumerate(calls):
            f()
            ev[k][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {name: [ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)]
             for i, (name, _) in enumerate(calls)}
    per_call = {name: float(np.mean(v)) for name, v in times.items()}
    spread = {name: (float(np.min(v)), float(np.max(v))) for name, v in times.items()}
    return wall, per_call, spread


def parse_smi(text):
    """Socket power (W) and the GFX clocks (MHz, one per XCD) from `amd-smi metric -p -c` text."""
    import re
    power = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clocks = [float(m.group(1)) for m in re.finditer(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    return (float(power.group(1)) if power else None), clocks


def power_sample(fn, ms_per_call, seconds=1.5):
    """Board power and GFX clock while fn runs back to back: ~`seconds` of calls are queued and
    amd-smi is read once while they run.  None when amd-smi is missing or fails."""
    import shutil
    import subprocess
    if shutil.which("amd-smi") is None:
        return None
    fn()
    torch.cuda.synchronize()
    for _ in range(max(8, int(seconds * 1e3 / max(ms_per_call, 1e-3)))):
        fn()
    time.sleep(min(0.5, seconds / 3))
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=30)
        text = r.stdout
    except (OSError, subprocess.SubprocessError):
        text = ""
    torch.cuda.synchronize()
    power, clocks = parse_smi(text)
    if power is None and not clocks:
        return None
    return {"socket_power_w": power, "gfx_clock_mhz_per_xcd": clocks,
            "gfx_clock_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None}


def run_gpu(s, steps, warmup, only=None):
    calls = s.calls()
    if only:
        calls = [c for c in calls if c[0] in only]
    wall, per_call, spread = run_calls(calls, steps, warmup)
    assert int(s.err.item()) == 0, "scatter reported an out-of-range block"
    return wall, per_call, spread


def host_info():
    """Host cores, CPU model and the NumPy / BLAS build the oracle runs on."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):                    # pragma: no cover
        info["affinity_cpus"] = None
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:                                      # pragma: no cover
        info["cpu_model"] = None
    info["numpy"] = np.__version__
    info["blas"] = None
    info["blas_threads"] = 1
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if libs:
            b = max(libs, key=lambda p: p.get("num_threads", 1))
            info["blas"] = f"{b.get('internal_api')} {b.get('version')} ({os.path.basename(b.get('filepath', ''))})"
            info["blas_threads"] = int(b.get("num_threads", 1))
    except Exception:                                    # pragma: no cover
        pass
    return info


def cpu_baseline(s):
    """The float64 oracle on a bounded sample of the same inputs, scaled to one step."""
    import oracle
    hi = host_info()
    blas = hi["blas_threads"]

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    c, m = s.rc, s.mc
    # about 15-30 s of oracle work on a 16-core host at either workload
    big = m["N"] > (1 << 19)
    L_r = min(8, c["L"])
    lg_m = 16 if big else 48
    blocks = 256
    t = {}
    t_sample = time.perf_counter()
    K = bits(s.K[:L_r])
    Mo = None
    for q in s.spans[:-1]:                               # the oracle's own session state
        Mo = oracle.qmem_update(bits(q), c["lam"], Mo)
    t0 = time.perf_counter()
    Mo = oracle.qmem_update(bits(s.spans[-1]), c["lam"], Mo)
    t["qmem"] = time.perf_counter() - t0
    M = Mo[:L_r]
    t0 = time.perf_counter()
    rule = oracle.rule_score(K, M, c["pi"], c["q_s"], c["q_e"])
    t["rule"] = (time.perf_counter() - t0) * c["L"] / L_r
    t0 = time.perf_counter()
    keep, _, _ = oracle.topk_select(rule, (0, c["pi"]), (c["q_s"], c["q_e"]), c["C"])
    oracle.slotmap_redirect(s.slots.cpu().numpy(), keep, c["dead_slot"])
    t["topk_slot"] = time.perf_counter() - t0
    # Mean-K on the first lg_m (layer, KV head) pairs
    G = m["H_q"] // m["H_kv"]
    LG = m["L"] * m["H_kv"]
    pairs = [(p // m["H_kv"], p % m["H_kv"]) for p in range(lg_m)]
    t0 = time.perf_counter()
    idx = [oracle.meank_build(bits(s.Kraw[l, g])[None, None])[0] for l, g in pairs]
    t["build"] = (time.perf_counter() - t0) * LG / lg_m
    t0 = time.perf_counter()
    R = np.zeros(s.nB)
    for (l, g), ix in zip(pairs, idx):
        R += oracle.meank_score(bits(s.Q[l, g * G:(g + 1) * G])[None], ix, m["n_sink"], m["n_recent"])
    t["score"] = (time.perf_counter() - t0) * LG / lg_m
    t0 = time.perf_counter()
    sel, _, _ = oracle.meank_select(R, m["n_sink"], m["n_recent"], m["budget"])
    t["select"] = time.perf_counter() - t0
    l, g = pairs[0]
    ks = bits(s.k_src[l, g])[None, None]
    vs = bits(s.v_src[l, g])[None, None]
    src = sel[:blocks] if s.src_block is None else np.arange(blocks)
    t0 = time.perf_counter()
    for _ in range(lg_m):
        oracle.rerope_scatter(ks, vs, src, None, m["pos_base"], m["theta"],
                              np.zeros((1, 1, 32 * blocks, m["D"])), np.zeros((1, 1, 32 * blocks, m["D"]), np.uint16))
    t["scatter"] = (time.perf_counter() - t0) * (LG / lg_m) * (s.n_sel / blocks)
    step = sum(t.values())
    tokens = c["N"] + m["N"]
    return {
        "value": tokens / step, "unit": "K-cache tokens/s", "cores": blas, "kind": "oracle",
        "sample": (f"float64 oracle on the same input bits: rule score over {L_r} of {c['L']} layers, "
                   f"Mean-K build and score over {lg_m} of {LG} (layer, KV head) pairs, re-RoPE scatter of "
                   f"{blocks} of {s.n_sel} blocks on {lg_m} pairs; each part scaled linearly to the full step "
                   f"({step:.1f} s extrapolated from {time.perf_counter() - t_sample:.1f} s of sampling). "
                   f"cores = the BLAS threads the float64 products use; elementwise numpy is single-threaded."),
        "host": hi,
        "seconds_per_step_extrapolated": step,
        "parts_s": {k: round(v, 3) for k, v in t.items()},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="rule-14b+meank-1m", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma-separated call names to time alone (profiling; not a headline figure). "
                         "Calls left out are not run, so a call that consumes another's output "
                         "(e.g. the scatter reading the Mean-K selection) sees whatever that buffer holds.")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the calls beyond the step (paged rule score, window score, "
                         "Mean-K append, working-set update)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run one 4 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--no-power-sample", action="store_true",
                    help="skip reading board power and clock with amd-smi (it starts a child process: "
                         "leave it out under a counter-collecting profiler)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs on one device and has no multi-GPU mode "
              "(sharding by (layer, KV head) is a design note). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    rule_name, meank_name = WORKLOADS[a.workload]
    log(f"[bench] setting up {a.workload}")
    s = Setup(rule_name, meank_name, dev)
    log(f"[bench] warmup {a.warmup}, timing {a.steps} steps")
    only = set(a.only.split(",")) if a.only else None
    wall, per_call, spread = run_gpu(s, a.steps, a.warmup, only)
    if only:
        print(json.dumps({"only": sorted(only), "ms_per_step": 1000.0 * wall / a.steps, "calls_ms": per_call,
                          "calls_ms_min_max": spread}))
        return
    ms_per_step = 1000.0 * wall / a.steps
    next_rows = None
    if not a.no_next_rows:
        log("[bench] timing the rows beyond the step")
        nr = NextRows(s, dev)
        _, nr_ms, nr_spread = run_calls(nr.calls(), a.steps, a.warmup)
        assert int(nr.err.item()) == 0, "working-set update rejected its input"
        next_rows = {}
        for name, ms in nr_ms.items():
            bound, amount = nr.work()[name]
            ach = amount / (ms * 1e-3) / 1e9
            next_rows[name] = {"ms": round(ms, 4), "ms_min": round(nr_spread[name][0], 4),
                               "ms_max": round(nr_spread[name][1], 4), "bound": bound, "achieved": round(ach, 2),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                               "per_launch": amount}
        next_rows["kvs_working_set_update"]["classes"] = {"moved": nr.n_moved, "incoming": nr.n_incoming,
                                                          "selected": int(nr.new.numel())}
        next_rows["kvs_window_score"]["window_rows"] = nr.W
        del nr
    # board power and clock while the dominant call runs back to back (after the timed steps)
    dom_call = max(per_call, key=lambda k: per_call[k])
    psample = None if a.no_power_sample else power_sample(dict(s.calls())[dom_call], per_call[dom_call])
    if a.copy_calibration:
        x = torch.empty(1 << 31, dtype=torch.int16, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    c, m = s.rc, s.mc
    tokens = c["N"] + m["N"]
    work = s.work()
    rows = {}
    for name, ms in per_call.items():
        bound, amount = work[name]
        if bound == "hbm":
            ach, peak, unit = amount / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        else:
            ach, peak, unit = amount / (ms * 1e-3) / 1e12, BF16_PEAK_TFLOPS, "TFLOP/s"
        rows[name] = {"ms": round(ms, 4), "ms_min": round(spread[name][0], 4), "ms_max": round(spread[name][1], 4),
                      "bound": bound, "achieved": round(ach, 2), "peak": peak,
                      "unit": unit, "frac": round(ach / peak, 4),
                      "per_launch": amount}
    traffic = measured_traffic(a.workload)
    for name, r in list(rows.items()) + list((next_rows or {}).items()):
        t = traffic.get(name)
        r["traffic"] = None if t is None else round(t)
    dom = max(rows, key=lambda k: rows[k]["ms"])
    d = rows[dom]
    turn = ("kvs_qmem_update", "kvs_rule_score", "kvs_topk_select_redirect[rule]")
    rule_ms = sum(per_call[k] for k in turn)
    rule_bytes = sum(work[k][1] for k in turn)
    # the eviction step alone (rule score, then top-k with the slot redirect), without the QueryMemory
    # update that precedes it in a turn
    select = ("kvs_rule_score", "kvs_topk_select_redirect[rule]")
    sel_ms = sum(per_call[k] for k in select)
    sel_bytes = sum(work[k][1] for k in select)
    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "K-cache tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "rule": {k: c[k] for k in ("L", "H_q", "H_kv", "D", "N", "pi", "q_s", "q_e", "C", "lam")},
                   "meank": {k: m[k] for k in ("L", "H_q", "H_kv", "D", "N", "Mq", "n_sink", "n_recent", "budget", "theta")},
                   "tokens_per_step": tokens},
        "roofline": {"call": dom, "kernels": " + ".join(k if isinstance(k, str) else " | ".join(k)
                                                         for k in call_kernels(a.workload).get(dom, [dom])),
                     "power_sample": psample,
                     "bound": d["bound"],
                     "achieved": d["achieved"], "peak": d["peak"], "unit": d["unit"], "frac": d["frac"],
                     "per_launch": d["per_launch"], "traffic": d["traffic"]},
        "rule_turn": {"ms": round(rule_ms, 4), "tokens_per_s": c["N"] / (rule_ms * 1e-3),
                      "hbm_gbps": rule_bytes / (rule_ms * 1e-3) / 1e9,
                      "frac_hbm_peak": rule_bytes / (rule_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "rule_select": {"ms": round(sel_ms, 4), "hbm_gbps": sel_bytes / (sel_ms * 1e-3) / 1e9,
                        "frac_hbm_peak": sel_bytes / (sel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "meank_score_tflops": rows["kvs_meank_score"]["achieved"],
        # the exact R_b runs two passes over the same tiles (row normalisers, then column sums), so
        # it executes twice the algorithmic flops; the mix ceiling is the rate a register-only loop
        # of the same MFMA 32x32x16 + exp2 epilogue mix sustains on all 256 CUs
        "meank_score_executed": {
            "tflop_per_call": 2 * work["kvs_meank_score"][1] / 1e12,
            "tflops": round(2 * rows["kvs_meank_score"]["achieved"], 2),
            "mix_ceiling_tflops": MIX_CEILING_TFLOPS,
            "frac_of_mix_ceiling": round(2 * rows["kvs_meank_score"]["achieved"] / MIX_CEILING_TFLOPS, 4),
            "random_operand_ceiling_tflops": MIX_CEILING_RANDOM_TFLOPS,
            "frac_of_random_operand_ceiling": round(2 * rows["kvs_meank_score"]["achieved"]
                                                    / MIX_CEILING_RANDOM_TFLOPS, 4)},
        "calls": rows,
        "next_rows": next_rows,
    }
    if not a.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded CPU sample")
        out["cpu_baseline"] = cpu_baseline(s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
