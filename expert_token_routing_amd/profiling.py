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
