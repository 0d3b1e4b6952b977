"""Turn rocprofv3 CSV output into the short summaries kept with the benchmark.

    python -m attention_space_retrieval_amd.rocprof_summary stats KERNEL_STATS_CSV --command CMD
        -> Markdown table of per-kernel durations (stdout)
    python -m attention_space_retrieval_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV --command CMD
        -> JSON with HBM bytes per dispatch for every library kernel (stdout)
    python -m attention_space_retrieval_amd.rocprof_summary counters COUNTER_CSV --kernel NAME ... --command CMD
        -> Markdown table of MFMA, VALU, exp2, clock and wait figures per named kernel, the mean over
           its dispatches, from one --pmc run of SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_INSTS_MFMA
           SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_WAIT_INST_ANY SQ_WAVE_CYCLES
           SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE (stdout)

The traffic summary scales the counters by what they read for the runtime's
own device copy of known size (bench.py --copy-calibration copies 4 GiB):
read factor = 4 GiB / (FETCH_SIZE KiB * 1024), write factor likewise with
WRITE_SIZE.  Each kernel's entry records a SHA-256 of the source that defines
it, so a reader can tell when the kernel has changed since the counters were
taken (bench.py then reports the traffic as null).
"""

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
HEADERS = ("kvs_internal.h", "rope_table.h")
COPY_BYTES = 1 << 32          # the 4 GiB calibration copy

# kernel name prefix -> source file that defines it
KERNEL_SOURCES = {
    "qmem_kernel": "qmem.hip",
    "rule_logits_mfma": "rule_score.hip", "rule_logits_f32": "rule_score.hip",
    "rule_lse_merge": "rule_score.hip", "rule_colsum": "rule_score.hip",
    "rule_fold_reset": "rule_score.hip", "rule_fold_queue": "rule_score.hip", "rule_fold_colsum": "rule_score.hip",
    "topk_wg_kernel": "topk.hip", "topk_stream_kernel": "topk.hip", "topk_mw_init": "topk.hip",
    "topk_mw_minmax": "topk.hip", "topk_mw_pass": "topk.hip", "topk_mw_count": "topk.hip",
    "topk_mw_emit": "topk.hip", "keep_all_kernel": "topk.hip",
    "slotmap_kernel": "topk.hip",
    "meank_build_raw": "meank_build.hip", "meank_build_derope": "meank_build.hip",
    "meank_append_kernel": "meank_build.hip",
    "meank_pass": "meank_score.hip", "meank_pass_dma": "meank_score.hip", "meank_reduce": "meank_score.hip",
    "meank_lse_merge": "meank_score.hip",
    "rerope_scatter_kernel": "rerope_scatter.hip", "v_scatter_kernel": "rerope_scatter.hip",
    "workset_diff": "workset.hip", "workset_apply": "workset.hip",
}


def short_name(full):
    """'void (anonymous namespace)::meank_pass<true>(unsigned short const*, ...)' -> 'meank_pass<true>'."""
    n = full.replace("(anonymous namespace)::", "")
    n = re.sub(r"^void ", "", n)
    depth, out = 0, []
    for ch in n:                      # cut at the argument list, keeping template arguments
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()


def base_name(short):
    return short.split("<")[0]


def source_hash(kernel_base):
    """SHA-256 over the kernel's source file and the shared device headers."""
    src = KERNEL_SOURCES.get(kernel_base)
    if src is None:
        return None
    h = hashlib.sha256()
    for f in (src,) + HEADERS:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def stats_markdown(path, command):
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["# rocprofv3 kernel statistics", "", "Command (repository root, one MI355X):", "",
             f"    {command}", "", "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = short_name(r["Name"])
        if name.startswith("at::") or name.startswith("__amd"):
            name = name[:60]
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.2f} |")
    return "\n".join(lines) + "\n"


def _per_dispatch(path, counter):
    """kernel short name -> list of counter values (KiB), one per dispatch, in dispatch order."""
    out = collections.defaultdict(list)
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r.get("Dispatch_Id", 0) or 0))
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def traffic_json(fetch_csv, write_csv, command):
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    copy = [k for k in f if k.startswith("__amd_rocclr_copyBuffer")]
    if not copy:
        raise SystemExit("no runtime copy dispatch found: run bench.py with --copy-calibration")
    fk = max(max(f[k]) for k in copy)            # the 4 GiB calibration copy is the largest
    wk = max(max(w.get(k, [0.0])) for k in copy)
    rf, wf = COPY_BYTES / (fk * 1024), COPY_BYTES / (wk * 1024)
    kernels = {}
    for name in sorted(set(f) | set(w)):
        b = base_name(name)
        if b not in KERNEL_SOURCES:
            continue
        fv, wv = f.get(name, []), w.get(name, [])
        kernels[name] = {
            "dispatches": len(fv),
            "fetch_kib_per_dispatch": fv,
            "write_kib_per_dispatch": wv,
            "read_bytes_mean": rf * 1024 * sum(fv) / max(1, len(fv)),
            "write_bytes_mean": wf * 1024 * sum(wv) / max(1, len(wv)),
            "source": KERNEL_SOURCES[b],
            "source_sha256": source_hash(b),
        }
    return {"command": command, "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": fk, "write_kib": wk,
                                                "read_factor": rf, "write_factor": wf},
            "kernels": kernels}


def counters_markdown(path, kernels, command, n_simd=1024, n_xcd=8):
    """Per-kernel means over the dispatches whose short name starts with one of `kernels`."""
    per = collections.defaultdict(dict)
    meta = {}
    for r in csv.DictReader(open(path)):
        name = short_name(r["Kernel_Name"])
        if not any(name.startswith(k) for k in kernels):
            continue
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = float(r["Counter_Value"])
        meta[d] = (name, int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    cols = collections.OrderedDict()
    for d in sorted(per):
        name, t0, t1 = meta[d]
        c, dur = per[d], (t1 - t0) * 1e-9
        cyc = c["GRBM_GUI_ACTIVE"] / n_xcd
        rows = cols.setdefault(name, collections.defaultdict(list))
        rows["dur"].append(dur * 1e3)
        rows["mfma"].append(c["SQ_INSTS_MFMA"])
        rows["trans"].append(c["SQ_INSTS_VALU_TRANS_F32"] * 64)
        rows["valu"].append(c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"])
        rows["clk"].append(cyc / dur / 1e9)
        rows["busy"].append(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * cyc))
        rows["coexec"].append(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"])
        rows["wait"].append(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"])
    mean = lambda v: sum(v) / len(v)
    names = list(cols)
    lines = ["Command (repository root, one MI355X):", "", f"    {command}", "",
             "| per dispatch (mean over " + ", ".join(f"{len(cols[n]['dur'])}" for n in names) + " dispatches) | "
             + " | ".join(f"`{n}`" for n in names) + " |", "|---" * (len(names) + 1) + "|"]
    def row(label, f):
        lines.append(f"| {label} | " + " | ".join(f(cols[n]) for n in names) + " |")
    row("duration (dispatch timestamps)", lambda c: f"{mean(c['dur']):.2f} ms ({min(c['dur']):.2f}-{max(c['dur']):.2f})")
    row("SQ_INSTS_MFMA", lambda c: f"{int(mean(c['mfma'])):,}")
    row("executed MFMA flops (32x32x16: 32768 each)", lambda c: f"{mean(c['mfma']) * 32768:.4e}")
    row("SQ_INSTS_VALU_TRANS_F32 x 64 lanes", lambda c: f"{mean(c['trans']):.4e}")
    row("SQ_INSTS_VALU per MFMA (the MFMA itself counted)", lambda c: f"{mean(c['valu']):.2f}")
    row("clock = GRBM_GUI_ACTIVE / XCDs / duration", lambda c: f"{mean(c['clk']):.2f} GHz ({min(c['clk']):.2f}-{max(c['clk']):.2f})")
    row("matrix cores busy = MFMA busy / (SIMDs x cycles)", lambda c: f"{100 * mean(c['busy']):.0f}%")
    row("VALU co-executing with the matrix cores", lambda c: f"{100 * mean(c['coexec']):.0f}%")
    row("SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES", lambda c: f"{100 * mean(c['wait']):.0f}%")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args(argv)
    if a.what == "counters":
        sys.stdout.write(counters_markdown(a.csv, a.kernel, a.command))
    elif a.what == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.command))
    else:
        json.dump(traffic_json(a.fetch_csv, a.write_csv, a.command), sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
