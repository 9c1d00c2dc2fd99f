"""Writes the oracle's whole-step velocities of the 32-block workloads, the
stored expected values of tests/test_gpu_fulldepth.py.

    python tests/golden/make_fulldepth_vel.py [--only NAME]

Calls only the oracle (oracle/dit.py) and the seeded input generators
(qi_synth); nothing here touches the HIP library.  For each case it runs one
joint DiT step (the DiT graph of the host contract, s.1) three times:
  exact     -- the definition in float64 (the oracle's default);
  bf16_f64  -- the bf16-compute reading (every matmul operand rounded once to
               bf16), float64 accumulation;
  bf16_f32  -- the same rounding points, float32 accumulation: a second
               legitimate order of the same bf16 arithmetic, whose distance to
               bf16_f64 is the cross-order spread that bf16 rounding alone
               produces through the stack.
Cases: the 384^2 workload (L 494, N 576) at sampler steps 0, 20 and 39, the
1024^2 workload (L 407, N 4096) and the 2048^2 workload (L 512, N 16384) at
step 20, and the 384^2 workload at step 20
with the shared modulation Linear (weight and bias) scaled by 1/4 and 1/8
(powers of two, so the scaled bf16 weights stay exact; the same weights
otherwise: a modulation closer to the identity, as in a trained DiT).  Step i
uses the timestep of the workload's 40-step schedule and the latent drawn
with seed 1234 + i, the other inputs the workload's own.

With --only NAME --mode MODE a single mode runs (the three can run in
separate processes); its velocity waits under tests/golden/_parts until the
last one completes the case's file.

Output: tests/golden/vel_<case>.npz with arrays exact, bf16_f64, bf16_f32
([N, 64] float32; the 2048^2 case: exact only, see CASE_MODES) and a JSON
string `meta`.  The 2048^2 case keeps every
fourth image token (the array `rows` lists them), which keeps the file near
the 1024^2 one in size; the metrics are then taken over those tokens."""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import qi_synth as qs  # noqa: E402
from oracle import dit  # noqa: E402

CASES = [
    # name, workload id, sampler step, modulation scale
    ("dit32-384px-step0", 3, 0, 1.0),
    ("dit32-384px-step20", 3, 20, 1.0),
    ("dit32-384px-step39", 3, 39, 1.0),
    ("dit32-384px-step20-mod0.25", 3, 20, 0.25),
    ("dit32-384px-step20-mod0.125", 3, 20, 0.125),
    ("dit32-1024px-step20", 4, 20, 1.0),
    ("dit32-2048px-step20", 5, 20, 1.0),
]
ROW_STRIDE = {"dit32-2048px-step20": 4}
# The 2048^2 case keeps the exact mode only: the bf16-compute reading rounds
# every attention probability (16384 x 16896 per head, 32 heads, 32 blocks),
# which takes the oracle several hours per mode on an 8-core host.
CASE_MODES = {"dit32-2048px-step20": ("exact",)}


def case_inputs(wl_id: int, step: int, mod_scale: float):
    """The case's workload, shared weights (fp32 values), inputs and t."""
    wl = qs.workload(wl_id)
    sw = qs.weights_as_f32(qs.shared_weights(wl, as_bf16=True))
    if mod_scale != 1.0:
        assert mod_scale in (0.5, 0.25, 0.125), "a power of two keeps the bf16 weights exact"
        sw = dict(sw)
        sw["w_mod"] = (sw["w_mod"].astype(np.float64) * mod_scale).astype(np.float32)
        sw["b_mod"] = (sw["b_mod"].astype(np.float64) * mod_scale).astype(np.float32)
    _, ts = dit.flow_sigmas(40, wl.N)
    t = dit.timestep_input(ts, step)
    return wl, sw, qs.img_tokens(wl, seed=qs.NOISE_SEED + step), qs.txt_feats(wl), t


MODES = (("exact", np.float64, False), ("bf16_f64", np.float64, True), ("bf16_f32", np.float32, True))
PARTS = os.path.join(HERE, "_parts")


def run_case(name, wl_id, step, mod_scale, only_mode=None):
    """Runs the case's modes (or only `only_mode`, whose velocity is kept
    under tests/golden/_parts until every mode of the case is there) and
    writes the case's file once all three are available."""
    wl, sw, X, E, t = case_inputs(wl_id, step, mod_scale)
    tc, tsn, ic, is_ = dit.rope_rows(wl.L, wl.h, wl.w)

    def blocks():
        for b in range(wl.n_blocks):
            yield qs.weights_as_f32(qs.block_weights(wl, b, as_bf16=True, threads=8))

    modes = CASE_MODES.get(name, tuple(m[0] for m in MODES))
    out = {}
    for mode, dtype, bf16 in MODES:
        part = os.path.join(PARTS, f"vel_{name}_{mode}.npy")
        if mode not in modes or (only_mode is not None and mode != only_mode):
            continue
        t0 = time.time()
        vel = dit.dit_step(sw, blocks, wl.L, X, E, t, tc, tsn, ic, is_, wl.heads, dtype=dtype, bf16=bf16)
        out[mode] = vel.astype(np.float32)
        print(f"{name} {mode}: {time.time() - t0:.0f} s", flush=True)
        if only_mode is not None:
            os.makedirs(PARTS, exist_ok=True)
            np.save(part, out[mode])
    for mode in modes:  # the modes other processes have finished
        part = os.path.join(PARTS, f"vel_{name}_{mode}.npy")
        if mode not in out and os.path.exists(part):
            out[mode] = np.load(part)
    if len(out) < len(modes):
        return
    stride = ROW_STRIDE.get(name, 1)
    if stride > 1:
        rows = np.arange(0, wl.N, stride)
        out = {k: v[rows] for k, v in out.items()}
        out["rows"] = rows.astype(np.int32)
    meta = {"case": name, "workload": wl.name, "sampler_step": step, "t": float(t), "mod_scale": mod_scale,
            "img_seed": qs.NOISE_SEED + step, "script": "tests/golden/make_fulldepth_vel.py", "row_stride": stride,
            "modes": list(modes)}
    if "bf16_f64" in out:
        meta["drift_bf16_vs_exact"] = dit.rel_l2(out["bf16_f64"], out["exact"])
        meta["spread_bf16_f32_vs_f64"] = dit.rel_l2(out["bf16_f32"], out["bf16_f64"])
    np.savez_compressed(os.path.join(HERE, f"vel_{name}.npz"), meta=json.dumps(meta), **out)
    for mode, _, _ in MODES:
        part = os.path.join(PARTS, f"vel_{name}_{mode}.npy")
        if os.path.exists(part):
            os.remove(part)
    print(json.dumps(meta), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", default=None)
    ap.add_argument("--mode", default=None, choices=[m[0] for m in MODES] + ["none"],
                    help="compute one mode of the --only case (modes can run in separate processes); "
                         "'none' only joins the finished modes into the case's file")
    args = ap.parse_args()
    if args.mode and not args.only:
        ap.error("--mode needs --only")
    for c in CASES:
        if args.only and c[0] != args.only:
            continue
        run_case(*c, only_mode=args.mode)


if __name__ == "__main__":
    main()
