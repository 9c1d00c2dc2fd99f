"""Parity of the 32-block step at full depth, block by block and whole-step.

Teacher-forced blocks (the method of the port page's gate table: the
reference's own input fed to every stage).  The oracle runs the joint step
of a workload through all 32 blocks in float64; before each block its
residual stream x_b is rounded to fp32 (the GPU's residual type) and that
same array is the input of both the oracle block and the GPU block
(qi_dit_block_fwd, joint pass, with the oracle's modulation rows).  Each
block's delta (output minus input) is compared over EVERY row:
  rel L2 <= 1e-2 over all rows, and the minimum over rows of the Pearson
  correlation of a row's delta over its H features >= 0.999.
Blocks 0 and 31 also run the image-only pass on the text K/V the joint pass
captured, which must equal the joint pass's image rows bit for bit.  Cases:
384^2 (L 494, N 576) at sampler steps 0, 20 and 39, and 1024^2 (L 407,
N 4096) at step 20.  At 2048^2 (L 512, N 16384) a teacher-forced trajectory
would hold the oracle on the test host for hours, so blocks 0, 15 and 31
take the oracle's embed output x_0 (block 0's true input) and are compared
on sampled rows.

Whole-step vel against the stored oracle velocities of
tests/golden/make_fulldepth_vel.py (exact, bf16-compute in float64 and in
float32 accumulation) at 384^2 and 1024^2, and the exact one at 2048^2 (on
every fourth image token, the rows the stored file keeps).  Through 32 random-init blocks bf16 rounding noise is
amplified beyond the 2e-2 bar (the bf16-compute oracle itself is that far
from the exact one), so the whole-step gate is: the GPU's distance to the
bf16-compute oracle is within 1.5x the spread between the two bf16 orders
(float32 vs float64 accumulation, same rounding points), and its correlation
with the exact oracle stays within the bf16 oracle's own.  With the shared
modulation scaled to 1/4 and 1/8 (a near-identity modulation, as in a
trained DiT) the bf16-compute oracle's own distance to the exact one falls
below the bar at 1/8, and there the exact-oracle 2e-2 / 0.999 bar itself is
gated.

Every figure is recorded by tests/parity_record.py."""
import json
import os

import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import assert_bits_equal, host, log
from tests.parity_record import record

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK_REL_BAR = 1e-2
BLOCK_CORR_BAR = 0.999
REL_L2_BAR = 2e-2
CORR_BAR = 0.999


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _row_corr_min(d, r):
    """Minimum over rows of the Pearson correlation of d[row] and r[row]."""
    d = d - d.mean(axis=1, keepdims=True)
    r = r - r.mean(axis=1, keepdims=True)
    num = np.sum(d * r, axis=1)
    den = np.sqrt(np.sum(d * d, axis=1) * np.sum(r * r, axis=1))
    return float(np.min(num / den))


def _delta_metrics(d_gpu, d_ref, L):
    err = d_gpu - d_ref
    row_rel = np.linalg.norm(err, axis=1) / np.linalg.norm(d_ref, axis=1)
    return {"rel": float(np.linalg.norm(err) / np.linalg.norm(d_ref)),
            "rel_text": float(np.linalg.norm(err[:L]) / np.linalg.norm(d_ref[:L])) if L else None,
            "rel_image": float(np.linalg.norm(err[L:]) / np.linalg.norm(d_ref[L:])),
            "corr_min": _row_corr_min(d_gpu, d_ref), "worst_row_rel": float(np.max(row_rel)),
            "worst_row": int(np.argmax(row_rel))}


def _inputs(m, wl, step):
    sw = qs.weights_as_f32(m["shared"])
    _, ts = dit.flow_sigmas(40, wl.N)
    t = dit.timestep_input(ts, step)
    X = qs.img_tokens(wl, seed=qs.NOISE_SEED + step)
    return sw, t, X, qs.txt_feats(wl)


def _teacher_forced(m, wl, step):
    import torch
    H, L, N = wl.hidden, wl.L, wl.N
    T = L + N
    dims, model = m["dims"], m["model"]
    sw, t, X, E = _inputs(m, wl, step)
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], t, H)
    x = dit.embed(sw, X, E)
    otc, ots, oic, ois = dit.rope_rows(L, wl.h, wl.w)
    ocos, osin = np.concatenate([otc, oic]), np.concatenate([ots, ois])
    tc, ts_, ic, is_ = qi.rope_tables(L, wl.h, wl.w)
    cos_d, sin_d = _dev(np.concatenate([tc, ic])), _dev(np.concatenate([ts_, is_]))
    ic_d, is_d = _dev(ic), _dev(is_)
    mod_d = _dev(np.stack([m_txt, m_img]).astype(np.float32))
    ws = qi.Workspace(dims, L, N)
    kv = torch.zeros(qi.kv_slot_elems(dims, L), dtype=torch.int16, device="cuda")
    xd = torch.empty((T, H), dtype=torch.float32, device="cuda")
    worst = {"rel": 0.0, "corr_min": 1.0}
    for b in range(wl.n_blocks):
        x_in = x.astype(np.float32)
        xd.copy_(torch.from_numpy(x_in))
        qi.dit_block_fwd(dims, model.block_struct(b), L, N, qi.QI_MODE_JOINT, xd, mod_d, cos_d, sin_d,
                         int(kv.data_ptr()), ws)
        x64 = x_in.astype(np.float64)
        x, _ = dit.dit_block(x64, L, qs.weights_as_f32(m["blocks"][b]), m_txt, m_img, ocos, osin, wl.heads)
        got = host(xd)
        assert np.all(np.isfinite(got)), f"block {b}: non-finite output"
        met = _delta_metrics(got.astype(np.float64) - x64, x - x64, L)
        if b in (0, wl.n_blocks - 1):
            xi = _dev(x_in[L:])
            qi.dit_block_fwd(dims, model.block_struct(b), L, N, qi.QI_MODE_IMAGE_ONLY, xi, mod_d, ic_d, is_d,
                             int(kv.data_ptr()), ws)
            assert_bits_equal(host(xi), got[L:], f"block {b}: image-only rows vs joint")
            met["image_only_bit_equal"] = True
        record("teacher_forced_block", workload=wl.name, sampler_step=step, block=b,
               x_rms=float(np.sqrt(np.mean(x64 * x64))), **met)
        worst["rel"] = max(worst["rel"], met["rel"])
        worst["corr_min"] = min(worst["corr_min"], met["corr_min"])
        assert met["rel"] <= BLOCK_REL_BAR and met["corr_min"] >= BLOCK_CORR_BAR, (b, met)
    record("teacher_forced_summary", workload=wl.name, sampler_step=step, blocks=wl.n_blocks,
           worst_rel=worst["rel"], worst_corr_min=worst["corr_min"])
    return dit.head(sw, x[L:])


def _gpu_step(m, wl, step, model=None):
    import torch
    _, t, X, E = _inputs(m, wl, step)
    rope = [_dev(a) for a in qi.rope_tables(wl.L, wl.h, wl.w)]
    ws = qi.Workspace(m["dims"], wl.L, wl.N)
    vel = torch.empty((wl.N, 64), dtype=torch.float32, device="cuda")
    qi.dit_step(model or m["model"], wl.L, wl.N, _dev(X), _dev(E), t, *rope, vel, ws)
    v = host(vel).copy()
    assert np.all(np.isfinite(v))
    return v


@pytest.mark.timeout(600)
@pytest.mark.parametrize("step", [0, 20, 39])
def test_teacher_forced_blocks_384px(model32, step):
    wl = qs.workload(3)
    log(f"teacher-forced 32 blocks at {wl.name}, sampler step {step}")
    vel_ref = _teacher_forced(model32, wl, step)
    vel = _gpu_step(model32, wl, step)
    record("whole_step_vs_exact_oracle_trajectory", workload=wl.name, sampler_step=step,
           rel=dit.rel_l2(vel, vel_ref), corr_min=dit.min_token_corr(vel, vel_ref))


@pytest.mark.timeout(900)
def test_teacher_forced_blocks_1024px(model32):
    wl = qs.workload(4)
    log(f"teacher-forced 32 blocks at {wl.name}, sampler step 20")
    vel_ref = _teacher_forced(model32, wl, 20)
    vel = _gpu_step(model32, wl, 20)
    record("whole_step_vs_exact_oracle_trajectory", workload=wl.name, sampler_step=20,
           rel=dit.rel_l2(vel, vel_ref), corr_min=dit.min_token_corr(vel, vel_ref))


@pytest.mark.timeout(600)
def test_blocks_2048px_sampled_rows(model32):
    """Blocks 0, 15 and 31 at 2048^2 on the oracle's embed output x_0 (block
    0's true input), against the oracle on sampled rows: first and last text
    and image rows, tile edges, random rows."""
    import torch
    wl = qs.workload(5)
    H, L, N = wl.hidden, wl.L, wl.N
    T = L + N
    dims, model = model32["dims"], model32["model"]
    sw, t, X, E = _inputs(model32, wl, 20)
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], t, H)
    x_in = dit.embed(sw, X, E).astype(np.float32)
    x64 = x_in.astype(np.float64)
    otc, ots, oic, ois = dit.rope_rows(L, wl.h, wl.w)
    tc, ts_, ic, is_ = qi.rope_tables(L, wl.h, wl.w)
    cos_d, sin_d = _dev(np.concatenate([tc, ic])), _dev(np.concatenate([ts_, is_]))
    mod_d = _dev(np.stack([m_txt, m_img]).astype(np.float32))
    ws = qi.Workspace(dims, L, N)
    kv = torch.zeros(qi.kv_slot_elems(dims, L), dtype=torch.int16, device="cuda")
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 63, 64, L - 1, L, L + 1, L + 255, L + 256, T - 257, T - 1] +
                      list(rng.integers(0, T, 13))))
    for b in (0, 15, 31):
        log(f"block {b} at {wl.name}")
        xd = _dev(x_in)
        qi.dit_block_fwd(dims, model.block_struct(b), L, N, qi.QI_MODE_JOINT, xd, mod_d, cos_d, sin_d,
                         int(kv.data_ptr()), ws)
        got = host(xd)[rows].astype(np.float64)
        ref = dit.dit_block_rows(x64, L, qs.weights_as_f32(model32["blocks"][b]), m_txt, m_img,
                                 np.concatenate([otc, oic]), np.concatenate([ots, ois]), wl.heads, rows)
        d_got, d_ref = got - x64[rows], ref - x64[rows]
        met = _delta_metrics(d_got, d_ref, int(np.sum(np.asarray(rows) < L)))
        record("sampled_rows_block", workload=wl.name, block=b, rows=len(rows), input="oracle embed x_0", **met)
        assert met["rel"] <= BLOCK_REL_BAR and met["corr_min"] >= BLOCK_CORR_BAR, (b, met)


def _golden(name):
    path = os.path.join(GOLDEN, f"vel_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (python tests/golden/make_fulldepth_vel.py)")
    z = np.load(path)
    g = {k: z[k] for k in ("exact", "bf16_f64", "bf16_f32") if k in z.files}
    g["rows"] = z["rows"] if "rows" in z.files else None
    return g, json.loads(str(z["meta"]))


def _scaled_shared(shared, s):
    """The shared weights with the modulation Linear scaled by the power of
    two s (exact on bf16 bits and fp32)."""
    sh = dict(shared)
    sh["w_mod"] = qs.f32_to_bf16_bits(qs.bf16_bits_to_f32(shared["w_mod"]) * np.float32(s))
    sh["b_mod"] = (shared["b_mod"].astype(np.float32) * np.float32(s)).astype(np.float32)
    return sh


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", ["dit32-384px-step0", "dit32-384px-step20", "dit32-384px-step39",
                                  "dit32-1024px-step20"])
def test_whole_step_vel_against_stored_oracle(model32, case):
    g, meta = _golden(case)
    wl = qs.workload({"384px": 3, "1024px": 4, "2048px": 5}[case.split("-")[1]])
    assert meta["workload"] == wl.name
    vel = _gpu_step(model32, wl, meta["sampler_step"])
    if g["rows"] is not None:
        vel = vel[g["rows"]]
    spread = dit.rel_l2(g["bf16_f32"], g["bf16_f64"])
    rec = record("whole_step_vel", case=case, workload=wl.name, sampler_step=meta["sampler_step"],
                 rel_vs_exact=dit.rel_l2(vel, g["exact"]), corr_vs_exact=dit.min_token_corr(vel, g["exact"]),
                 rel_vs_bf16=dit.rel_l2(vel, g["bf16_f64"]), corr_vs_bf16=dit.min_token_corr(vel, g["bf16_f64"]),
                 bf16_oracle_rel_vs_exact=dit.rel_l2(g["bf16_f64"], g["exact"]),
                 bf16_oracle_corr_vs_exact=dit.min_token_corr(g["bf16_f64"], g["exact"]),
                 bf16_cross_order_spread=spread)
    assert rec["rel_vs_bf16"] <= 1.5 * spread, rec
    assert rec["corr_vs_exact"] >= 1.0 - 1.5 * (1.0 - rec["bf16_oracle_corr_vs_exact"]), rec


@pytest.mark.timeout(300)
def test_whole_step_vel_2048px_against_exact_oracle(model32):
    """The 2048^2 step (L 512, N 16384, all 32 blocks) against the exact
    oracle on every fourth image token.  Its stored file holds the exact mode
    only (the bf16-compute reading is too slow on the oracle's host at this
    size), so there is no cross-order spread to gate on; the gate is the
    bf16-compute oracle's own full-depth distance to the exact one measured at
    384^2 and 1024^2 (rel L2 5.3e-2 to 7.3e-2, token correlation >= 0.992),
    with margin: rel L2 <= 0.1 and correlation >= 0.99."""
    g, meta = _golden("dit32-2048px-step20")
    wl = qs.workload(5)
    assert meta["workload"] == wl.name and g["rows"] is not None
    vel = _gpu_step(model32, wl, meta["sampler_step"])[g["rows"]]
    rec = record("whole_step_vel", case="dit32-2048px-step20", workload=wl.name,
                 sampler_step=meta["sampler_step"], tokens=int(len(g["rows"])),
                 rel_vs_exact=dit.rel_l2(vel, g["exact"]), corr_vs_exact=dit.min_token_corr(vel, g["exact"]))
    assert rec["rel_vs_exact"] <= 0.1 and rec["corr_vs_exact"] >= 0.99, rec


@pytest.mark.timeout(300)
@pytest.mark.parametrize("scale", [0.25, 0.125])
def test_whole_step_vel_near_identity_modulation(model32, scale):
    """The same 32 blocks at 384^2 with the shared modulation Linear scaled
    by 1/4 and 1/8 (scale and gate rows closer to zero, as in a trained DiT).
    The bf16-compute oracle's own distance to the exact one falls with the
    scale (2.1e-2 at 1/4, 1.6e-2 at 1/8); the GPU must stay within 1.5x the
    bf16 cross-order spread of the bf16 oracle and no farther from the exact
    oracle than 1.25x the bf16 oracle is.  Where the bf16 reading itself
    meets the 2e-2 / 0.999 bar (1/8), the GPU must meet it too."""
    case = f"dit32-384px-step20-mod{scale}"
    g, meta = _golden(case)
    assert meta["mod_scale"] == scale
    wl = qs.workload(3)
    model = model32["model"].with_shared(_scaled_shared(model32["shared"], scale))
    vel = _gpu_step(model32, wl, 20, model=model)
    spread = dit.rel_l2(g["bf16_f32"], g["bf16_f64"])
    rec = record("whole_step_vel", case=case, workload=wl.name, sampler_step=20, mod_scale=scale,
                 rel_vs_exact=dit.rel_l2(vel, g["exact"]), corr_vs_exact=dit.min_token_corr(vel, g["exact"]),
                 rel_vs_bf16=dit.rel_l2(vel, g["bf16_f64"]), corr_vs_bf16=dit.min_token_corr(vel, g["bf16_f64"]),
                 bf16_oracle_rel_vs_exact=dit.rel_l2(g["bf16_f64"], g["exact"]),
                 bf16_oracle_corr_vs_exact=dit.min_token_corr(g["bf16_f64"], g["exact"]),
                 bf16_cross_order_spread=spread)
    assert rec["rel_vs_bf16"] <= 1.5 * spread, rec
    assert rec["rel_vs_exact"] <= 1.25 * rec["bf16_oracle_rel_vs_exact"], rec
    if rec["bf16_oracle_rel_vs_exact"] <= REL_L2_BAR and rec["bf16_oracle_corr_vs_exact"] >= CORR_BAR:
        assert rec["rel_vs_exact"] <= REL_L2_BAR and rec["corr_vs_exact"] >= CORR_BAR, rec
    else:
        assert scale == 0.25, "the bf16 reading is expected to meet the bar at 1/8"
