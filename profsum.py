"""Summarise rocprofv3 CSV output into short text profiles.

Usage (after the rocprofv3 runs named in each mode's docstring)::

    python3 profsum.py stats    KERNEL_STATS.csv  --command "..."
    python3 profsum.py trace    KERNEL_TRACE.csv  --command "..."
    python3 profsum.py traffic  FETCH.csv WRITE.csv COPY_FETCH.csv \
        COPY_WRITE.csv --copy-bytes 1073741824 --workload llama128k --budget 0.1 --tau 8 \
        --command "..."
    python3 profsum.py counters COUNTERS.csv --command "..." \
        [--workload llama128k --budget 0.1 --tau 8]

Each mode prints Markdown.  The traffic mode also prints one
``bench-traffic: {json}`` line per attention kernel, which ``bench.py`` reads
back to fill the roofline's ``traffic`` field, and the counters mode with a
workload one ``bench-mfma: {json}`` line per attention kernel (its MfmaUtil),
both only while the digest of the attention kernel's sources still matches
the one recorded with the counters (a changed kernel invalidates them).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

# measurement tooling beside bench.py, not part of the library
PKG_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_sparse_long_kap_amd")
ATTN_SOURCES = ("csrc/attn_fwd.hip", "csrc/cosa_internal.h", "csrc/cosa_api.hip")


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that editing a comment
    does not count as changing the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def attention_source_digest(read=None) -> str:
    """sha256 over the code (comments dropped) of the sources that decide what
    the attention kernel does.  ``read(rel)`` may supply the text of a file."""
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        if read is None:
            with open(os.path.join(PKG_DIR, rel)) as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(rel.encode() + b"\0" + _code_only(text).encode() + b"\0")
    return h.hexdigest()[:16]


def entry_of(kernel: str):
    """C entry point that launches an attention kernel instance, from the last
    template argument (the page-walk mode), or None for other kernels."""
    if re.search(r"attn_dense_pp_kernel<", kernel):
        return "cosa_dense_prefill"
    m = re.search(r"attn_fwd_kernel<\s*\d+,\s*\d+,\s*(\w+)\s*(?:,\s*\d+\s*)*>", kernel)
    if not m:
        return None
    return {"0": "cosa_dense_prefill", "false": "cosa_dense_prefill",
            "1": "cosa_osk_prefill", "true": "cosa_osk_prefill",
            "2": "cosa_block_mask_prefill"}.get(m.group(1))


def short_name(kernel: str) -> str:
    s = kernel
    if "::" in s:
        s = s.split("(anonymous namespace)::")[-1]
    return re.sub(r"\((cosa::)?\w+Params\)$", "", s)


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _workgroups(r):
    """Workgroups of a dispatch record (None when the CSV has no sizes)."""
    if "Grid_Size" not in r or "Workgroup_Size" not in r:
        return None
    return int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))


def per_kernel_counter(path):
    """{((kernel, workgroups), counter): [values per dispatch]} from a
    counter_collection CSV: launches of one kernel over different parts of
    the work (the chunks of the fused call) are kept apart."""
    agg = collections.defaultdict(list)
    for r in _rows(path):
        agg[((r["Kernel_Name"], _workgroups(r)), r["Counter_Name"])].append(
            float(r["Counter_Value"]))
    return agg


def _label(kw):
    k, wg = kw
    return f"`{short_name(k)}`" + ("" if wg is None else f" | {wg}")


def stats_md(path, command):
    out = ["| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in _rows(path):
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e6:.4f} | {float(r['MinNs']) / 1e6:.4f} | "
                   f"{float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.2f}% |")
    return "\n".join([f"Command: `{command}`", "", *out])


def trace_md(path, command):
    """Per-dispatch kernel times grouped by (kernel, grid size): launches of
    one kernel over different parts of the work are kept apart."""
    agg = collections.defaultdict(list)
    for r in _rows(path):
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) *
               int(r["Grid_Size_Z"]) // max(1, int(r["Workgroup_Size_X"]) *
                                            int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])))
        agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    out = ["| kernel | workgroups | calls | avg ms | median ms | min ms | max ms | total ms |",
           "|---|---|---|---|---|---|---|---|"]
    for (k, wg), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        srt = sorted(v)
        med = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] +
                                                               srt[len(srt) // 2])
        out.append(f"| `{k}` | {wg} | {len(v)} | {sum(v) / len(v):.4f} | {med:.4f} | "
                   f"{min(v):.4f} | {max(v):.4f} | {sum(v):.3f} |")
    return "\n".join([f"Command: `{command}`", "", *out])


def _copy_kib(path, counter):
    """Largest per-dispatch value of ``counter`` for the device copy kernel."""
    best = 0.0
    for ((k, _), c), v in per_kernel_counter(path).items():
        if c == counter and "copyBuffer" in k:
            best = max(best, max(v))
    if best <= 0:
        raise SystemExit(f"no copy dispatch with {counter} in {path}")
    return best


def traffic_md(fetch, write, cfetch, cwrite, copy_bytes, workload, budget, tau, command):
    f_scale = copy_bytes / (_copy_kib(cfetch, "FETCH_SIZE") * 1024.0)
    w_scale = copy_bytes / (_copy_kib(cwrite, "WRITE_SIZE") * 1024.0)
    fr, wr = per_kernel_counter(fetch), per_kernel_counter(write)
    digest = attention_source_digest()
    lines = [f"Command: `{command}`", "",
             f"Copy calibration ({copy_bytes} B device copy): FETCH_SIZE x{f_scale:.3f}, "
             f"WRITE_SIZE x{w_scale:.3f} to reach true bytes.", "",
             "| kernel | workgroups | dispatches | FETCH KiB (raw) | WRITE KiB (raw) | "
             "read GB (scaled) | written GB (scaled) | total GB |",
             "|---|---|---|---|---|---|---|---|"]
    records = []
    for (kw, c), v in sorted(fr.items(), key=lambda kv: (kv[0][0][0], -(kv[0][0][1] or 0))):
        k, wg = kw
        if c != "FETCH_SIZE" or "cosa" not in k:
            continue
        wv = wr.get((kw, "WRITE_SIZE"))
        if not wv:
            continue
        fk, wk = sum(v) / len(v), sum(wv) / len(wv)
        rd, wt = fk * 1024 * f_scale, wk * 1024 * w_scale
        lines.append(f"| `{short_name(k)}` | {wg} | {len(v)} | {fk:.6g} | {wk:.6g} | "
                     f"{rd / 1e9:.3f} | {wt / 1e9:.3f} | {(rd + wt) / 1e9:.3f} |")
        if "attn_fwd_kernel" in k:
            records.append({"kernel": short_name(k), "entry": entry_of(k), "workgroups": wg,
                            "workload": workload, "budget": budget,
                            "tau": tau, "read_bytes": round(rd), "write_bytes": round(wt),
                            "bytes_per_launch": round(rd + wt), "source_digest": digest})
    lines.append("")
    lines += ["bench-traffic: " + json.dumps(r) for r in records]
    return "\n".join(lines)


def counters_md(path, command, xcds=8, simds=1024, workload=None, budget=None, tau=None):
    """Per-dispatch means per (kernel, grid size) and the MfmaUtil of each
    where the pass holds its counters; with a workload, one ``bench-mfma``
    line per attention kernel, which bench.py reads back while the attention
    sources still match the recorded digest."""
    agg = per_kernel_counter(path)
    records = []
    digest = attention_source_digest() if workload is not None else None
    kernels = sorted({kw for kw, _ in agg if "cosa" in kw[0]},
                     key=lambda kw: (kw[0], -(kw[1] or 0)))
    names = sorted({c for _, c in agg})
    out = [f"Command: `{command}`", "",
           "| kernel | workgroups | " + " | ".join(names) + " | MfmaUtil |",
           "|---|---|" + "---|" * (len(names) + 1)]
    for k in kernels:
        vals = {c: sum(agg[(k, c)]) / len(agg[(k, c)]) for c in names if (k, c) in agg}
        util = ""
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and vals.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE is summed over the XCDs; busy cycles over the SIMDs
            u = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (vals["GRBM_GUI_ACTIVE"] / xcds * simds)
            util = f"{u:.3f}"
            if workload is not None and entry_of(k[0]) is not None:
                records.append({"kernel": short_name(k[0]), "entry": entry_of(k[0]),
                                "workgroups": k[1], "workload": workload, "budget": budget,
                                "tau": tau, "mfma_util": round(u, 4), "source_digest": digest})
        out.append(f"| `{short_name(k[0])}` | {k[1]} | " +
                   " | ".join(f"{vals[c]:.4g}" if c in vals else "" for c in names) +
                   f" | {util} |")
    if records:
        out.append("")
        out += ["bench-mfma: " + json.dumps(r) for r in records]
    return "\n".join(out)


def read_mfma_util(path, workload, budget, tau, entry):
    """MfmaUtil recorded for the whole-layer launch (largest grid) of the kernel
    behind ``entry`` with these settings, or None when absent or taken on
    different kernel sources."""
    if not os.path.exists(path):
        return None
    digest = attention_source_digest()
    best = None
    with open(path) as f:
        for line in f:
            if not line.startswith("bench-mfma: "):
                continue
            r = json.loads(line[len("bench-mfma: "):])
            if (r.get("entry") == entry and r["workload"] == workload and
                    abs(r["budget"] - budget) < 1e-9 and abs(r["tau"] - tau) < 1e-9 and
                    r["source_digest"] == digest):
                if best is None or (r.get("workgroups") or 0) > (best.get("workgroups") or 0):
                    best = r
    return best


def read_traffic(path, workload, budget, tau):
    """Bytes per launch recorded for the whole-layer attention launch with these
    settings (the largest grid of cosa_osk_prefill's kernel), or None when
    absent or taken on different kernel sources."""
    if not os.path.exists(path):
        return None
    digest = attention_source_digest()
    best = None
    with open(path) as f:
        for line in f:
            if not line.startswith("bench-traffic: "):
                continue
            r = json.loads(line[len("bench-traffic: "):])
            if (r.get("entry") == "cosa_osk_prefill" and r["workload"] == workload and
                    abs(r["budget"] - budget) < 1e-9 and abs(r["tau"] - tau) < 1e-9 and
                    r["source_digest"] == digest):
                if best is None or (r.get("workgroups") or 0) > (best.get("workgroups") or 0):
                    best = r
    return best


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch")
    t.add_argument("write")
    t.add_argument("copy_fetch")
    t.add_argument("copy_write")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--budget", type=float, required=True)
    t.add_argument("--tau", type=float, required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--command", required=True)
    c.add_argument("--workload")
    c.add_argument("--budget", type=float)
    c.add_argument("--tau", type=float)
    a = ap.parse_args(argv)
    if a.mode == "stats":
        print(stats_md(a.csv, a.command))
    elif a.mode == "trace":
        print(trace_md(a.csv, a.command))
    elif a.mode == "traffic":
        print(traffic_md(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.workload,
                         a.budget, a.tau, a.command))
    else:
        print(counters_md(a.csv, a.command, workload=a.workload, budget=a.budget, tau=a.tau))
    return 0


if __name__ == "__main__":
    sys.exit(main())
