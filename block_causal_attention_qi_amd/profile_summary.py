"""Summaries of rocprofv3 runs of bench.py, written to profiles/.

    python -m block_causal_attention_qi_amd.profile_summary trace DIR
    python -m block_causal_attention_qi_amd.profile_summary traffic DIR
    python -m block_causal_attention_qi_amd.profile_summary mfma DIR

DIR holds the CSV output of the commands that each summary names (run from
the repository root on one MI355X; see TRACE_CMD, TRAFFIC_CMDS, MFMA_CMD).
Kernel launches are classified by name and launch order into the kinds of the
library's own timer (the two residual-epilogue GEMMs share one instantiation:
the one right after attention is the output projection), and by the step they
belong to into the image-only and joint passes (label_launches).  The JSON
sidecars carry the hash of the kernel sources they were measured on, so
bench.py can tell when they no longer describe the current kernels."""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("common.hpp", "gemm.hpp", "attention_args.hpp", "attention.hpp", "elementwise.hpp")

BENCH_ARGS = "python -u bench.py --steps 10 --warmup 1 --no-cpu-baseline --no-cfg --no-encoder --no-workloads"
TRACE_CMD = f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o bench -- {BENCH_ARGS}"
TRAFFIC_CMDS = [f"rocprofv3 --pmc {c} --output-format csv -d DIR/{c} -o bench -- {BENCH_ARGS}"
                for c in ("FETCH_SIZE", "WRITE_SIZE")] + \
               [f"rocprofv3 --pmc {c} --output-format csv -d DIR/{c}_copy -o copy -- python -u bench.py --calibrate-copy"
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
MFMA_CMD = ("rocprofv3 --pmc SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVES "
            f"--output-format csv -d DIR/MFMA -o bench -- {BENCH_ARGS}")


def kernel_code_text(src: str) -> str:
    """Kernel sources without comments, whitespace runs collapsed (a comment
    edit changes no kernel)."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_sha256() -> str:
    csrc = os.path.join(PKG, "csrc")
    src = "".join(open(os.path.join(csrc, f)).read() for f in KERNEL_SOURCES)
    return hashlib.sha256(kernel_code_text(src).encode()).hexdigest()


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def kind_of(name: str, prev: str | None) -> str:
    import re
    m = re.search(r"gemm_bf16_(?:large_|mid_|lds_)?kernel<(\d)", name)
    if m:
        epi = int(m.group(1))  # the epilogue: 0 fp32 store, 1 residual, 2 SwiGLU, 3 QKV
        if epi == 2:
            return "gemm_gate_up"
        if epi == 3:
            return "gemm_qkv"
        if epi == 1:  # the output projection follows attention (its row tail follows it)
            return "gemm_o" if prev in ("attention", "gemm_o") else "gemm_down"
        return "gemm_txt"
    for key, kind in (("attn", "attention"), ("rmsnorm", "norm_mod"), ("head_kernel", "head"),
                      ("mod_gemv", "modulation"), ("img_embed", "img_embed"), ("euler", "euler")):
        if key in name:
            return kind
    return "other"


def label_launches(names):
    """(kind, pass) of each launch of a bench run, in launch order.  Every DiT
    step starts with its modulation kernel; a step that runs the text
    projection is a joint pass (its text norm and text projection are the
    "joint (text)" launches), every other step an image-only pass.  (A joint
    pass may split a GEMM into a 256-row-tile head and a row tail, so launch
    shapes alone do not tell the passes apart.)"""
    kinds, prev = [], None
    for n in names:
        k = kind_of(n, prev)
        kinds.append(k)
        prev = k
    starts = [i for i, k in enumerate(kinds) if k == "modulation"] + [len(kinds)]
    passes = ["other"] * len(kinds)
    for s0, s1 in zip(starts, starts[1:]):
        step = kinds[s0:s1]
        joint = "gemm_txt" in step
        txt_end = s0 + step.index("gemm_txt") if joint else s0
        for i in range(s0, s1):
            if not joint:
                passes[i] = "image-only"
            elif kinds[i] == "gemm_txt" or (kinds[i] == "norm_mod" and i < txt_end):
                passes[i] = "joint (text)"
            else:
                passes[i] = "joint"
    return list(zip(kinds, passes))


def summarize_trace(d: str):
    st = _rows(os.path.join(d, "trace", "bench_kernel_stats.csv"))
    tr = sorted(_rows(os.path.join(d, "trace", "bench_kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    agg = collections.defaultdict(list)
    for r, (k, p) in zip(tr, label_launches([r["Kernel_Name"] for r in tr])):
        g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r.get("Grid_Size_Z", 1) or 1)
        agg[(k, p, g)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    cmd = TRACE_CMD.replace("DIR", "OUT")
    lines = ["# Kernel trace: 32-block DiT at 1024^2 (L 407, N 4096), bench loop", "",
             "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
             "Summary written by `python -m block_causal_attention_qi_amd.profile_summary trace OUT` (OUT: the runs' output directory).",
             "", "rocprofv3 kernel_stats (all launches of the run, joint and image-only steps):", "",
             "| kernel | calls | avg us | share % |", "|---|---|---|---|"]
    for r in st[:12]:
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    lines += ["", "Per kernel kind and launch shape (grid = work-items); the image-only rows are the",
              "launches bench.py's `kernels` and `roofline` entries average:", "",
              "| kind | grid | launches | avg us | min us | max us | pass |", "|---|---|---|---|---|---|---|"]
    kinds = {}
    for (k, p, g), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        if k == "other" or p == "other":
            continue
        lines.append(f"| {k} | {g} | {len(v)} | {statistics.mean(v):.1f} | {min(v):.1f} | {max(v):.1f} | {p} |")
        # the pass's main launch shape (a joint pass may add a row-tail launch)
        if p not in kinds.setdefault(k, {}):
            kinds[k][p] = {"grid": g, "launches": len(v), "avg_us": round(statistics.mean(v), 2),
                           "median_us": round(statistics.median(v), 2)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "dit32_1024px_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    out = {"what": "average launch duration per kernel kind and pass from rocprofv3 --kernel-trace",
           "command": cmd, "kernel_source_sha256": kernel_source_sha256(),
           "kernel_source_sha256_of": " ".join(KERNEL_SOURCES) + ", comments removed and whitespace collapsed",
           "kinds": kinds}
    with open(os.path.join(PROFILES, "dit32_1024px_kernel_trace.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


def _pmc(path):
    """Counter values per (kind, pass, grid) of a one-counter rocprofv3 run."""
    rows = sorted(_rows(path), key=lambda x: int(x["Dispatch_Id"]))
    vals = collections.defaultdict(list)
    for x, (k, p) in zip(rows, label_launches([x["Kernel_Name"] for x in rows])):
        vals[(k, p, int(x["Grid_Size"]))].append(float(x["Counter_Value"]))
    return vals


def summarize_traffic(d: str):
    fetch = _pmc(os.path.join(d, "FETCH_SIZE", "bench_counter_collection.csv"))
    write = _pmc(os.path.join(d, "WRITE_SIZE", "bench_counter_collection.csv"))

    def copy_kib(sub):
        v = [float(x["Counter_Value"]) for x in _rows(os.path.join(d, sub, "copy_counter_collection.csv"))]
        return statistics.mean([a for a in v if a > 1e5])
    cfv, cwv = copy_kib("FETCH_SIZE_copy"), copy_kib("WRITE_SIZE_copy")
    gib_kib = (1 << 30) / 1024
    sf, sw = gib_kib / cfv, gib_kib / cwv
    out = {"what": "HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), "
                   "scaled by the same counters read on a 1 GiB device copy",
           "commands": [c.replace("DIR", "OUT") for c in TRAFFIC_CMDS],
           "copy_calibration": {"bytes_each_way": 1 << 30, "fetch_kib": cfv, "write_kib": cwv,
                                "fetch_scale": sf, "write_scale": sw},
           "kernel_source_sha256": kernel_source_sha256(),
           "kernel_source_sha256_of": " ".join(KERNEL_SOURCES) + ", comments removed and whitespace collapsed",
           "kernels": {}}
    for (k, p, g), v in sorted(fetch.items(), key=lambda kv: -len(kv[1]) * statistics.mean(kv[1])):
        if k == "other" or p == "other" or len(v) < 4:
            continue
        if p in out["kernels"].get(k, {}):  # the pass's main launch shape only
            continue
        w = write.get((k, p, g), [0.0])
        out["kernels"].setdefault(k, {})[p] = {
            "grid": g, "launches": len(v), "fetch_kib": statistics.mean(v), "write_kib": statistics.mean(w),
            "hbm_bytes": statistics.mean(v) * 1024 * sf + statistics.mean(w) * 1024 * sw}
    with open(os.path.join(PROFILES, "dit32_1024px_hbm_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["kernels"], indent=1))


def summarize_mfma(d: str):
    path = os.path.join(d, "MFMA", "bench_counter_collection.csv")
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    rows = sorted(_rows(path), key=lambda x: (int(x["Dispatch_Id"]), x["Counter_Name"]))
    ids = sorted({int(x["Dispatch_Id"]) for x in rows})
    first = {}
    for x in rows:
        first.setdefault(int(x["Dispatch_Id"]), x["Kernel_Name"])
    label = dict(zip(ids, label_launches([first[i] for i in ids])))
    for x in rows:
        k, p = label[int(x["Dispatch_Id"])]
        vals[(k, p, int(x["Grid_Size"]))][x["Counter_Name"]].append(float(x["Counter_Value"]))
    cmd = MFMA_CMD.replace("DIR", "OUT")
    lines = ["# MFMA busy per kernel: 32-block DiT at 1024^2 (L 407, N 4096)", "",
             "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
             "Summary written by `python -m block_causal_attention_qi_amd.profile_summary mfma OUT` (OUT: the runs' output directory).", "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES): the share of the",
             "cycles in which the CUs run the kernel that each SIMD's matrix core is busy, whatever the",
             "clock.  SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 against the kernel's algorithmic FLOPs checks",
             "that no masked or padded MFMA work is counted as useful.", "",
             "| kind | pass | grid | launches | MFMA busy | MOPS x 512 / launch (TFLOP) |", "|---|---|---|---|---|---|"]
    for (k, p, g), dd in sorted(vals.items(), key=lambda kv: -sum(kv[1].get("SQ_BUSY_CU_CYCLES", [0]))):
        if k == "other" or p == "other" or not dd.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            continue
        busy = statistics.mean(dd["SQ_VALU_MFMA_BUSY_CYCLES"]) / (4 * statistics.mean(dd["SQ_BUSY_CU_CYCLES"]))
        mops = statistics.mean(dd.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) * 512 / 1e12
        if busy < 0.01:
            continue
        lines.append(f"| {k} | {p} | {g} | {len(dd['SQ_WAVES'])} | {busy:.3f} | {mops:.3f} |")
    with open(os.path.join(PROFILES, "dit32_1024px_mfma_busy.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    what, d = sys.argv[1], sys.argv[2]
    {"trace": summarize_trace, "traffic": summarize_traffic, "mfma": summarize_mfma}[what](d)
