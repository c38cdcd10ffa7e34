"""Summaries of rocprofv3 output for the layer's kernels.

Turns the CSV files of two kinds of rocprofv3 runs into the short text
summaries kept under ``profiles/``:

* ``--kernel-trace --stats``: average duration and share of each kernel
  (``<name>_kernel_stats.csv``);
* ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one counter per run):
  HBM bytes per dispatch, scaled by what the same counters report for a
  plain device copy of known size (``<name>_counter_collection.csv``);
* ``--pmc`` passes of matrix-core, cache and wave counters (names from
  ``rocprofv3 -L`` on gfx950): MFMA busy cycles against the SIMDs' active
  cycles, MFMA operations issued, L2 hit rate, L1-to-L2 read latency, LDS
  bank conflicts and wave waiting time per dispatch;
* ``--hip-trace --hsa-trace --memory-allocation-trace --kernel-trace`` of
  ``tests/steady_state_child.py``: the HIP and HSA calls, allocations and
  dispatches between the child's two marker calls (steady-state forwards).

Kernels are keyed by the pipeline stage they implement, so a reader (such as
bench.py's roofline) can find the bytes of "gate_up" whichever kernel
variant ran it.

Usage::

    python -m lora_expert_gemm_amd.profiling stats <workload> <stats.csv> <out.md> <command...>
    python -m lora_expert_gemm_amd.profiling traffic <workload> <fetch.csv> <write.csv> \
        <copy_fetch.csv> <copy_write.csv> <copy_mib> <traffic.json> <out.md> <source_hash> <command...>
    python -m lora_expert_gemm_amd.profiling steady <trace dir> <out.md> <command...>
    python -m lora_expert_gemm_amd.profiling mfma <workload> <out.md> <csv>... -- <command...>

The trailing words are the rocprofv3 command(s) that made the CSVs, recorded
in the summary; a ";;" word separates commands.
"""
import csv
import json
import os
import re
import sys
from collections import defaultdict

# kernel name prefix -> pipeline stage (first match wins)
_STAGES = [
    ("k_route_align_small", "route_align"),
    ("k_route", "route_align"),
    ("k_align", "route_align"),
    ("k_tiled_shrink<false", "shrink_gate_up"),
    ("k_tiled_shrink<true", "shrink_down"),
    ("k_shrink<", None),  # resolved from the FROM_H template argument below
    ("k_tiled8<true", "gate_up"),
    ("k_tiled8<false", "down"),
    ("k_tiled<true", "gate_up"),
    ("k_tiled<false", "down"),
    ("k_gate_up", "gate_up"),
    ("k_down", "down"),
    ("k_combine", "combine"),
]


def short_name(name):
    """'void moelora::(anonymous namespace)::k_x<a, b>(moelora::GemmArgs)' -> 'k_x<a, b>'."""
    m = re.search(r"(k_[a-z_0-9]+(<[^()]*>)?)", name)
    return m.group(1) if m else name.strip()


def stage_of(kernel):
    k = short_name(kernel)
    for prefix, stage in _STAGES:
        if k.startswith(prefix):
            if stage is None:  # k_shrink<DT, TG, VEC, EVEN_K, FROM_H, waves>
                return "shrink_down" if k.rstrip(">").split(",")[4].strip() == "true" \
                    else "shrink_gate_up"
            return stage
    return None


def read_stats(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append(dict(kernel=short_name(r["Name"]), calls=int(r["Calls"]),
                             avg_us=float(r["AverageNs"]) / 1e3, share=float(r["Percentage"])))
    return rows


def read_counter(path, counter):
    """Mean value of `counter` per dispatch, per kernel (short name)."""
    tot, n = defaultdict(float), defaultdict(int)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = short_name(r["Kernel_Name"])
            tot[k] += float(r["Counter_Value"])
            n[k] += 1
    return {k: tot[k] / n[k] for k in tot}, dict(n)


def write_stats_md(workload, stats_csv, out_md, command):
    rows = read_stats(stats_csv)
    lines = [f"# Kernel durations: {workload}", "",
             "Command (run from /tmp with TMPDIR=/tmp):", "", "```", command, "```", "",
             "| kernel | stage | calls | average (us) | share |", "|---|---|---|---|---|"]
    for r in rows:
        k = r["kernel"]
        if stage_of(k) is None and len(k) > 80:  # library kernels: the name's start
            k = k[:77] + "..."
        lines.append(f"| {k} | {stage_of(r['kernel']) or '-'} | {r['calls']} | "
                     f"{r['avg_us']:.2f} | {r['share']:.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows


def write_traffic(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib,
                  traffic_json, out_md, source_hash, command):
    fetch, nf = read_counter(fetch_csv, "FETCH_SIZE")
    write, _ = read_counter(write_csv, "WRITE_SIZE")
    cf, _ = read_counter(copy_fetch_csv, "FETCH_SIZE")
    cw, _ = read_counter(copy_write_csv, "WRITE_SIZE")
    kib = copy_mib * 1024.0
    copy_kernel = max(cf, key=cf.get)  # the copy dominates its run
    fs, ws = kib / cf[copy_kernel], kib / cw[copy_kernel]
    entry = {}  # stage -> summed over the kernels that make up the stage
    for k in fetch:
        st = stage_of(k)
        if st is None:
            continue
        b = (fetch[k] * fs + write.get(k, 0.0) * ws) * 1024.0
        e = entry.setdefault(st, dict(kernel="", fetch_kib=0.0, write_kib=0.0, bytes=0.0))
        e["kernel"] = (e["kernel"] + " + " if e["kernel"] else "") + k
        e["fetch_kib"] += fetch[k]
        e["write_kib"] += write.get(k, 0.0)
        e["bytes"] += b
    t = {}
    if os.path.exists(traffic_json):
        with open(traffic_json) as f:
            t = json.load(f)
    if t.get("kernel_source") != source_hash:
        t = {"kernel_source": source_hash, "workloads": {}}
    t["fetch_scale"], t["write_scale"] = fs, ws
    t["workloads"][workload] = entry
    with open(traffic_json, "w") as f:
        json.dump(t, f, indent=1)
    lines = [f"# HBM traffic counters: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; one counter per pass):", "", "```",
             command, "```", "",
             f"Kernel code: `{source_hash}` (sha256 prefix over the device-kernel sources with "
             "comments and whitespace removed, as bench.py computes it).", "",
             f"Calibration: a plain {copy_mib} MiB device copy ({copy_kernel}) reports "
             f"FETCH_SIZE = {cf[copy_kernel]:.0f} KiB and WRITE_SIZE = {cw[copy_kernel]:.0f} KiB "
             f"per dispatch, so FETCH_SIZE is scaled by {fs:.4f} and WRITE_SIZE by {ws:.4f}.", "",
             "| stage | kernel | dispatches | FETCH_SIZE (KiB, mean) | WRITE_SIZE (KiB, mean) "
             "| scaled HBM bytes / launch |", "|---|---|---|---|---|---|"]
    for st, v in entry.items():
        disp = nf.get(v["kernel"].split(" + ")[0], 0)
        lines.append(f"| {st} | {v['kernel']} | {disp} | {v['fetch_kib']:.0f} "
                     f"| {v['write_kib']:.0f} | {v['bytes'] / 1e6:.1f} MB |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return entry


# gfx950 (MI355X): 8 XCDs of 32 CUs, 4 SIMDs per CU.  GRBM_GUI_ACTIVE is
# reported summed over the XCDs, SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs.
N_XCD, N_SIMD = 8, 1024
MFMA_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "TCC_HIT_sum", "TCC_MISS_sum", "TCP_TCC_READ_REQ_LATENCY_sum",
                 "TCP_TCC_READ_REQ_sum", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                 "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")


def write_mfma(workload, csvs, out_md, command):
    """Matrix-core utilisation and memory-side counters per stage."""
    vals, dur = defaultdict(dict), defaultdict(list)
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                if stage_of(k) is None or r["Counter_Name"] not in MFMA_COUNTERS:
                    continue
                vals[k].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    mean = lambda k, c: (sum(vals[k][c]) / len(vals[k][c])) if vals[k].get(c) else None
    lines = [f"# Matrix-core and memory counters: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp; one counter set per pass):", "", "```",
             command, "```", "",
             f"Per dispatch means.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
             f"{N_XCD} x {N_SIMD} SIMDs); MFMA TFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the "
             "matrix-core work issued, padding rows and columns included); L2 hit = TCC_HIT / "
             "(TCC_HIT + TCC_MISS); L1->L2 latency = TCP_TCC_READ_REQ_LATENCY / "
             "TCP_TCC_READ_REQ (cycles per request); waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES.  "
             "Durations are those of the counter runs (slower than unprofiled ones).", "",
             "| stage | kernel | dispatches | MFMA busy | MFMA TFLOP / launch | L2 hit "
             "| L1->L2 latency | LDS bank conflicts / LDS active | waiting |",
             "|---|---|---|---|---|---|---|---|---|"]
    pct = lambda x: "-" if x is None else f"{100 * x:.1f}%"
    for k in sorted(vals, key=lambda k: -(mean(k, "GRBM_GUI_ACTIVE") or 0)):
        g, busy = mean(k, "GRBM_GUI_ACTIVE"), mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        mops = mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        hit, miss = mean(k, "TCC_HIT_sum"), mean(k, "TCC_MISS_sum")
        lat, req = mean(k, "TCP_TCC_READ_REQ_LATENCY_sum"), mean(k, "TCP_TCC_READ_REQ_sum")
        bc, la = mean(k, "SQ_LDS_BANK_CONFLICT"), mean(k, "SQ_LDS_IDX_ACTIVE")
        wa, wc = mean(k, "SQ_WAIT_ANY"), mean(k, "SQ_WAVE_CYCLES")
        util = busy / (g / N_XCD * N_SIMD) if g and busy is not None else None
        lines.append(
            f"| {stage_of(k)} | {k} | {len(vals[k].get('GRBM_GUI_ACTIVE', []))} | {pct(util)} | "
            f"{'-' if mops is None else f'{mops * 512 / 1e12:.3f}'} | "
            f"{pct(hit / (hit + miss)) if hit is not None and miss and hit + miss > 0 else '-'} | "
            f"{'-' if not req else f'{lat / req:.0f}'} | "
            f"{pct(bc / la) if la else '-'} | {pct(wa / wc) if wc else '-'} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


# Calls that load code or allocate: none may fall between the markers.
CODE_OR_MEMORY = ("hsa_executable_create", "hsa_executable_load", "hsa_executable_freeze",
                  "hsa_code_object", "hsa_memory_allocate", "hsa_amd_memory_pool_allocate",
                  "hsa_amd_memory_lock", "hipModule", "hipMalloc", "hipHostMalloc", "hipFree",
                  "hipHostRegister", "__hipRegister")
MARKER = "hipDriverGetVersion"


def _csv(trace_dir, suffix):
    for root, _, files in os.walk(trace_dir):
        for f in files:
            if f.endswith(suffix):
                with open(os.path.join(root, f)) as fh:
                    return list(csv.DictReader(fh))
    return []


def steady_window(trace_dir):
    """Counts of HIP / HSA calls, allocations and dispatches before the first
    marker call and between the two markers of the steady-state child."""
    hip = _csv(trace_dir, "_hip_api_trace.csv")
    hsa = _csv(trace_dir, "_hsa_api_trace.csv")
    mem = _csv(trace_dir, "_memory_allocation_trace.csv")
    ker = _csv(trace_dir, "_kernel_trace.csv")
    marks = sorted(int(r["Start_Timestamp"]) for r in hip if r["Function"] == MARKER)
    if len(marks) != 2:
        raise ValueError(f"expected two {MARKER} markers, found {len(marks)}")
    a, b = marks

    def split(rows, key):
        before, inside = defaultdict(int), defaultdict(int)
        for r in rows:
            t = int(r["Start_Timestamp"])
            if t < a:
                before[r[key]] += 1
            elif t < b and r[key] != MARKER:
                inside[r[key]] += 1
        return dict(before), dict(inside)

    out = {}
    out["hip_before"], out["hip_inside"] = split(hip, "Function")
    out["hsa_before"], out["hsa_inside"] = split(hsa, "Function")
    out["alloc_before"], out["alloc_inside"] = split(mem, "Operation")
    kb, ki = split(ker, "Kernel_Name")
    out["kernels_before"] = {short_name(k): v for k, v in kb.items()}
    out["kernels_inside"] = {short_name(k): v for k, v in ki.items()}
    out["forbidden_inside"] = {k: v for d in (out["hip_inside"], out["hsa_inside"])
                               for k, v in d.items() if k.startswith(CODE_OR_MEMORY)}
    return out


def write_steady_md(trace_dir, out_md, command):
    w = steady_window(trace_dir)
    lines = ["# Steady-state forwards: code loads, allocations and API calls", "",
             "One plan of a 128-expert top-8 layer (H 2048, I 768, 32 adapters of rank 16, "
             "bf16) serves forwards at 1, 3, 24, 40, 64, 100, 256, 300, 700, 1024 and 2048 "
             "tokens (16-, 32- and 64-row streaming blocks, row- and tile-wise LoRA, 128-row "
             "LDS-tiled blocks).  The first forward runs before the first marker call; the "
             "other 21 forwards run between the two markers (`tests/steady_state_child.py`).",
             "", "Command (run from /tmp with TMPDIR=/tmp):", "", "```", command, "```", ""]

    def table(title, d):
        lines.extend([f"**{title}**", "", "| call | count |", "|---|---|"])
        for k, v in sorted(d.items(), key=lambda kv: -kv[1]):
            lines.append(f"| {k} | {v} |")
        if not d:
            lines.append("| (none) | 0 |")
        lines.append("")

    table("Code-object loads and allocations between the markers", w["forbidden_inside"])
    table("Memory allocations between the markers", w["alloc_inside"])
    table("HIP API calls between the markers", w["hip_inside"])
    table("HSA API calls between the markers", w["hsa_inside"])
    loads = {k: v for k, v in w["hsa_before"].items()
             if k.startswith(("hsa_executable_load", "hsa_code_object"))}
    table("Code-object loads before the first marker (start-up and the first forward)", loads)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return w


def main(argv):
    # command words; a ";;" word starts a new command line
    def cmd(words):
        return " ".join(words).replace(" ;; ", "\n")
    if argv[0] == "stats":
        write_stats_md(argv[1], argv[2], argv[3], cmd(argv[4:]))
    elif argv[0] == "mfma":
        i = argv.index("--")
        write_mfma(argv[1], argv[3:i], argv[2], cmd(argv[i + 1:]))
    elif argv[0] == "steady":
        write_steady_md(argv[1], argv[2], cmd(argv[3:]))
    elif argv[0] == "traffic":
        (wl, fcsv, wcsv, cfcsv, cwcsv, mib, tj, md, h), rest = argv[1:10], argv[10:]
        write_traffic(wl, fcsv, wcsv, cfcsv, cwcsv, float(mib), tj, md, h, cmd(rest))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
