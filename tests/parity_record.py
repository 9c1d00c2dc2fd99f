"""Measured parity figures of the GPU tests, kept as a record.

Each call appends one JSON line to records.jsonl in the directory named by
QI_PARITY_RECORD_DIR (default: qi_parity_records in the system's temporary
directory) and prints it, so the figures a test gates on survive the run and
the long tests show progress.  tests/records/ keeps the records of a full
`python -m pytest tests -m gpu` run and their summary (summarize below)."""
from __future__ import annotations

import json
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD_DIR = os.environ.get("QI_PARITY_RECORD_DIR") or os.path.join(tempfile.gettempdir(), "qi_parity_records")


def record(kind: str, **fields) -> dict:
    rec = {"kind": kind, "time": round(time.time(), 1), **fields}
    line = json.dumps(rec, default=float)
    try:
        os.makedirs(RECORD_DIR, exist_ok=True)
        with open(os.path.join(RECORD_DIR, "records.jsonl"), "a") as f:
            f.write(line + "\n")
    except OSError:  # a read-only tree still runs the test
        pass
    print(line, flush=True)
    sys.stdout.flush()
    return rec


def summarize(path: str) -> str:
    """Markdown tables of a records.jsonl: per-workload teacher-forced worst
    blocks, sampled-row blocks and whole-step velocities (the latest record of
    each kind and key wins)."""
    recs = [json.loads(line) for line in open(path) if line.strip()]
    out = [f"Parity records from `{os.path.basename(path)}` ({len(recs)} records), written by the GPU tests of",
           "`python -m pytest tests -m gpu` (tests/parity_record.py) on one MI355X; this summary by",
           f"`python tests/parity_record.py {os.path.basename(path)}`.", ""]
    tf = {}
    for r in recs:
        if r["kind"] == "teacher_forced_block":
            tf[(r["workload"], r["sampler_step"], r["block"])] = r
    if tf:
        out += ["## Teacher-forced blocks (all rows; bar rel <= 1e-2, corr_min >= 0.999)", "",
                "| workload | sampler step | blocks | worst rel (block) | median rel | worst corr_min (block) "
                "| worst text rel | worst image rel |", "|---|---|---|---|---|---|---|---|"]
        for wl, st in sorted({(k[0], k[1]) for k in tf}):
            rs = [tf[k] for k in sorted(tf) if k[0] == wl and k[1] == st]
            wr = max(rs, key=lambda r: r["rel"])
            wc = min(rs, key=lambda r: r["corr_min"])
            rels = sorted(r["rel"] for r in rs)
            txt = [r["rel_text"] for r in rs if r.get("rel_text") is not None]
            out.append(f"| {wl} | {st} | {len(rs)} | {wr['rel']:.3e} ({wr['block']}) | {rels[len(rels) // 2]:.3e} "
                       f"| {wc['corr_min']:.6f} ({wc['block']}) | {max(txt) if txt else float('nan'):.3e} "
                       f"| {max(r['rel_image'] for r in rs):.3e} |")
        out.append("")
    sr = {(r["workload"], r["block"]): r for r in recs if r["kind"] == "sampled_rows_block"}
    if sr:
        out += ["## Sampled-row blocks on the oracle's embed output", "",
                "| workload | block | rows | rel | corr_min |", "|---|---|---|---|---|"]
        for k in sorted(sr):
            r = sr[k]
            out.append(f"| {k[0]} | {k[1]} | {r['rows']} | {r['rel']:.3e} | {r['corr_min']:.6f} |")
        out.append("")
    ws = {r["case"]: r for r in recs if r["kind"] == "whole_step_vel"}
    if ws:
        out += ["## Whole-step vel against the stored oracle velocities", "",
                "| case | rel vs exact | corr vs exact | rel vs bf16 oracle | bf16 oracle rel vs exact "
                "| bf16 cross-order spread |", "|---|---|---|---|---|---|"]
        def e3(r, f):  # the exact-only cases (2048^2) have no bf16-oracle fields
            return f"{r[f]:.3e}" if f in r else "—"

        for k in sorted(ws):
            r = ws[k]
            out.append(f"| {k} | {r['rel_vs_exact']:.3e} | {r['corr_vs_exact']:.6f} | {e3(r, 'rel_vs_bf16')} "
                       f"| {e3(r, 'bf16_oracle_rel_vs_exact')} | {e3(r, 'bf16_cross_order_spread')} |")
        out.append("")
    tr = {(r["workload"], r["sampler_step"]): r for r in recs if r["kind"] == "whole_step_vs_exact_oracle_trajectory"}
    if tr:
        out += ["## Whole-step vel of the teacher-forced runs against the exact oracle's own trajectory", "",
                "| workload | sampler step | rel | corr_min |", "|---|---|---|---|"]
        for k in sorted(tr):
            r = tr[k]
            out.append(f"| {k[0]} | {k[1]} | {r['rel']:.3e} | {r['corr_min']:.6f} |")
        out.append("")
    return "\n".join(out)


if __name__ == "__main__":
    # python tests/parity_record.py RECORDS.jsonl > SUMMARY.md
    print(summarize(sys.argv[1]))
