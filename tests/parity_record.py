"""Measured parity figures of the GPU tests, kept as a record.

Each call appends one JSON line to gpurun_out/parity/records.jsonl (under the
repository root; the folder the GPU runs bring back) and prints it, so the
figures a test gates on survive the run and the long tests show progress."""
from __future__ import annotations

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORD_DIR = os.path.join(ROOT, "gpurun_out", "parity")


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
