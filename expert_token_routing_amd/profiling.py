"""Reading rocprofv3 output and the committed profile summaries.

``summarize`` turns a rocprofv3 output directory (kernel stats, or counter
collection) into a short markdown summary for ``profiles/``.  Each summary
ends with one JSON line (``<!-- occ-profile {...} -->``) that ``bench.py``
reads back: the HBM traffic of a kernel measured with FETCH_SIZE /
WRITE_SIZE, scaled by the same counters' reading for a plain copy kernel of
known size, and the hash of the kernel source it was measured on (a stale
figure -- source changed since -- is reported as null).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "expert_token_routing_amd", "csrc")
TAG = re.compile(r"<!-- occ-profile (\{.*\}) -->")


def source_sha(filename: str) -> str:
    with open(os.path.join(CSRC, filename), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def find(pattern_dir: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))


def kernel_stats(out_dir: str) -> list[dict]:
    rows = []
    for p in find(out_dir, "kernel_stats.csv"):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    return rows


def counter_rows(out_dir: str) -> list[dict]:
    rows = []
    for p in find(out_dir, "counter_collection.csv"):
        with open(p) as f:
            rows += list(csv.DictReader(f))
    return rows


def short_name(kernel: str) -> str:
    m = re.search(r"(k_[a-z0-9_]+)", kernel)
    if m:
        return m.group(1)
    return kernel.split("(")[0][-60:]


def counters_by_kernel(rows: list[dict], counter: str) -> dict[str, list[float]]:
    """Per-dispatch values of `counter`, grouped by kernel short name."""
    by: dict[str, dict[str, float]] = {}
    for r in rows:
        name = r.get("Counter_Name") or r.get("Counter-Name") or ""
        if name != counter:
            continue
        kern = short_name(r.get("Kernel_Name") or r.get("Kernel-Name") or "")
        disp = r.get("Dispatch_Id") or r.get("Dispatch-Id") or str(len(by))
        val = float(r.get("Counter_Value") or r.get("Counter-Value") or 0)
        by.setdefault(kern, {}).setdefault(disp, 0.0)
        by[kern][disp] += val
    return {k: list(v.values()) for k, v in by.items()}


def committed(kernel: str, workload: str) -> dict | None:
    """The machine-readable record for (kernel, workload) in profiles/, if any."""
    for p in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(p):
            m = TAG.search(line)
            if not m:
                continue
            rec = json.loads(m.group(1))
            if rec.get("kernel") == kernel and rec.get("workload") == workload:
                return rec
    return None


def traffic_bytes(kernel: str, workload: str, source: str) -> float | None:
    """Scaled HBM bytes per launch (fetch + write), or None when absent/stale."""
    rec = committed(kernel, workload)
    if not rec or "fetch_bytes" not in rec or "write_bytes" not in rec:
        return None
    if rec.get("src_sha") != source_sha(source):
        return None
    return float(rec["fetch_bytes"]) + float(rec["write_bytes"])


def _fmt_ns(ns: float) -> str:
    return f"{ns / 1e3:.1f}"


def summarize_stats(out_dir: str, command: str, title: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    rows = kernel_stats(out_dir)
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {_fmt_ns(float(r['AverageNs']))} | "
                     f"{_fmt_ns(float(r['MinNs']))} | {_fmt_ns(float(r['MaxNs']))} | "
                     f"{float(r['Percentage']):.2f} |")
    return "\n".join(lines) + "\n"


def summarize_traffic(fetch_dir: str, write_dir: str, fetch_cmd: str, write_cmd: str,
                      workload: str, copy_bytes: int, sources: dict[str, str],
                      title: str) -> str:
    """HBM traffic per dispatch from FETCH_SIZE / WRITE_SIZE passes, scaled by
    the reading for a plain device copy of `copy_bytes` (the largest
    copyBuffer dispatches of the run)."""
    fr, wr = counter_rows(fetch_dir), counter_rows(write_dir)

    def per_kernel(rows, counter):
        by: dict[str, list[tuple[float, str]]] = {}
        for r in rows:
            if (r.get("Counter_Name") or "") != counter:
                continue
            name = r.get("Kernel_Name") or ""
            key = "copy" if "copyBuffer" in name else short_name(name)
            by.setdefault(key, []).append(float(r.get("Counter_Value") or 0) * 1024.0)
        return by

    f, w = per_kernel(fr, "FETCH_SIZE"), per_kernel(wr, "WRITE_SIZE")
    big = lambda xs: [x for x in xs if x >= 0.5 * copy_bytes]
    fc, wc = big(f.get("copy", [])), big(w.get("copy", []))
    if not fc or not wc:
        raise RuntimeError("no calibration copy found in the counter runs")
    f_scale = copy_bytes / (sum(fc) / len(fc))
    w_scale = copy_bytes / (sum(wc) / len(wc))
    lines = [f"# {title}", "", "Commands (run from the repository root on one MI355X):", "",
             "```", fetch_cmd, write_cmd, "```", "",
             f"Calibration: a plain device copy of {copy_bytes} bytes reads "
             f"{sum(fc) / len(fc):.4g} B (FETCH_SIZE) and writes {sum(wc) / len(wc):.4g} B "
             f"(WRITE_SIZE); scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| kernel | dispatches | fetch MB / dispatch | write MB / dispatch |",
             "|---|---|---|---|"]
    recs = []
    for k in sorted(set(f) | set(w)):
        if k == "copy" or not k.startswith("k_"):
            continue  # the calibration copy and the harness's own torch kernels
        fv, wv = f.get(k, [0.0]), w.get(k, [0.0])
        fb, wb = f_scale * sum(fv) / len(fv), w_scale * sum(wv) / len(wv)
        lines.append(f"| {k} | {len(fv)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
        if k in sources:
            recs.append({"kernel": k, "workload": workload, "fetch_bytes": round(fb),
                         "write_bytes": round(wb), "src_sha": source_sha(sources[k]),
                         "source": sources[k]})
    lines.append("")
    for rec in recs:
        lines.append(f"<!-- occ-profile {json.dumps(rec)} -->")
    return "\n".join(lines) + "\n"


def agent_info(out_dir: str) -> dict:
    """The GPU agent's row of a rocprofv3 run (SIMD, CU and XCC counts)."""
    for p in find(out_dir, "agent_info.csv"):
        with open(p) as f:
            for r in csv.DictReader(f):
                if r.get("Agent_Type") == "GPU":
                    return r
    return {}


def summarize_counters(out_dirs: list[str], commands: list[str], title: str,
                       kernels: list[str] | None = None) -> str:
    """Markdown table of per-dispatch counter means for the GEMM kernels and
    the rates derived from them: the clock (GRBM_GUI_ACTIVE per XCC over the
    dispatch's duration), the share of SIMD cycles the matrix pipes were
    busy (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCC times the
    SIMDs), LDS bank conflicts per LDS access cycle and the share of wave
    cycles spent waiting on counters (s_waitcnt)."""
    info = agent_info(out_dirs[0])
    simds, xcc = int(info.get("Simd_Count", 1024)), int(info.get("Num_Xcc", 8))
    vals: dict[str, dict[str, list[float]]] = {}
    dur: dict[str, dict[tuple, int]] = {}
    for i, d in enumerate(out_dirs):
        for r in counter_rows(d):
            k = short_name(r["Kernel_Name"])
            if kernels and k not in kernels:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.setdefault(k, {})[(i, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) -
                                                            int(r["Start_Timestamp"]))
    mean = lambda v: sum(v) / len(v) if v else None
    lines = [f"# {title}", "", "Commands (run from the repository root on one MI355X):", "", "```"]
    lines += commands + ["```", "",
                         f"GPU: {simds} SIMDs in {xcc} XCCs. Counters are per dispatch, averaged; the "
                         "dispatches of a counter run are serialized and slower than in a timed run.", "",
                         "| kernel | dispatches per run | avg us | clock GHz | matrix pipes busy % | "
                         "LDS bank conflicts per access % | wave cycles waiting % |",
                         "|---|---|---|---|---|---|---|"]
    order = sorted(vals, key=lambda k: -sum(dur[k].values()))
    for k in order:
        c = {n: mean(v) for n, v in vals[k].items()}
        us = mean(list(dur[k].values())) / 1e3
        gui = c.get("GRBM_GUI_ACTIVE")
        clk = gui / xcc / (us * 1e3) if gui else None
        busy = (100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / xcc * simds)
                if gui and c.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None else None)
        bank = (100 * c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
                if c.get("SQ_LDS_IDX_ACTIVE") else None)
        wait = (100 * c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
                if c.get("SQ_WAVE_CYCLES") else None)
        f = lambda x, fmt: "—" if x is None else fmt.format(x)
        lines.append(f"| {k} | {len(dur[k]) // len(out_dirs)} | {us:.1f} | {f(clk, '{:.2f}')} | {f(busy, '{:.1f}')} | "
                     f"{f(bank, '{:.2f}')} | {f(wait, '{:.1f}')} |")
    return "\n".join(lines) + "\n"


def _main(argv=None):
    import argparse

    ap = argparse.ArgumentParser(description="Summarize rocprofv3 output for profiles/")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--fetch-command", required=True)
    t.add_argument("--write-command", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--title", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--kernels", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        text = summarize_counters(a.dirs, a.command, a.title,
                                  [k for k in a.kernels.split(",") if k] or None)
    elif a.cmd == "stats":
        text = summarize_stats(a.dir, a.command, a.title)
    else:
        sources = {"k_gemm_up": "gemm_bf16.hip", "k_gemm_down": "gemm_bf16.hip",
                   "k_gemm_up_m128": "gemm_bf16.hip", "k_gemm_down_m128": "gemm_bf16.hip",
                   "k_gemm_up_dense": "gemm_bf16.hip", "k_gemm_down_dense": "gemm_bf16.hip",
                   "k_gemm_up_f32": "gemm_f32.hip", "k_gemm_down_f32": "gemm_f32.hip",
                   "k_gate_bf16": "gate.hip", "k_sim_gram": "similarity.hip",
                   "k_dispatch": "rows.hip", "k_combine": "rows.hip",
                   "k_merge_slots": "rows.hip",
                   "k_route": "route.hip", "k_route_rows": "route.hip",
                   "k_brim_fill": "brim.hip", "k_brim_small": "brim.hip"}
        text = summarize_traffic(a.fetch_dir, a.write_dir, a.fetch_command, a.write_command,
                                 a.workload, a.copy_bytes, sources, a.title)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    _main()
