"""GPU parity of the first-block cache (Fast mode of [MLX] "Optional modes";
reading S21: block 0 always runs, blocks 1.. are skipped while block 0's
residual changes less than the threshold against the last full step, a
skipped step adding that step's residual of blocks 1..):

  - threshold 0 never skips: every step equals the ordinary cached step bit
    for bit;
  - a step repeated on identical inputs is skipped (decided on the device) and
    reproduces the full step up to fp32 rounding;
  - a denoising loop against the oracle's, teacher-forced (each oracle step
    takes the GPU loop's latents, so only the step's own error is compared):
    the same skip decisions at thresholds chosen from the oracle's own change
    values, away from them, and each step's vel within the parity bar.

Workloads: the reduced block with 3 blocks and the full-width block with 3
blocks (2 in the loop, where the bar holds for two full-width blocks), so
there are blocks to skip."""
import math

import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import GpuWorkload, assert_bits_equal, host, log

pytestmark = pytest.mark.gpu

REL_L2_BAR = 2e-2
CORR_BAR = 0.999


def _setup(wl_id, n_blocks=3):
    wl = qs.workload(wl_id, n_blocks=n_blocks)
    g = GpuWorkload(wl)
    cache = g.new_cache()
    g.capture(np.float32(0.95), cache)
    fbc = qi.FirstBlockCache(g.dims, wl.N)
    return wl, g, cache, fbc


def _fbc_step(g, cache, fbc, t, threshold):
    qi.dit_step_fbc(g.model, g.L, g.N, g.img, t, g.rope[2], g.rope[3], cache, threshold, fbc, g.vel, g.ws)
    return host(g.vel).copy()


@pytest.mark.parametrize("wl_id", [1, 2])
def test_threshold_zero_equals_cached_steps(wl_id):
    wl, g, cache, fbc = _setup(wl_id)
    for k, t in enumerate((0.8, 0.6, 0.6, 0.55)):
        g.set_inputs(qs.img_tokens(wl, seed=40 + (k % 2)), None)
        got = _fbc_step(g, cache, fbc, np.float32(t), 0.0)
        ref = host(g.step(np.float32(t), cache=cache)).copy()
        assert_bits_equal(got, ref, f"threshold 0, step {k}")
    s = fbc.stats()
    assert s["steps"] == 4 and s["skipped"] == 0


@pytest.mark.parametrize("wl_id", [1, 2])
def test_repeated_step_is_skipped(wl_id):
    wl, g, cache, fbc = _setup(wl_id)
    g.set_inputs(qs.img_tokens(wl, seed=61), None)
    t = np.float32(0.7)
    v1 = _fbc_step(g, cache, fbc, t, 0.08)
    s = fbc.stats()
    assert s["skipped"] == 0 and math.isinf(s["last_change"])
    v2 = _fbc_step(g, cache, fbc, t, 0.08)
    s = fbc.stats()
    assert s["steps"] == 2 and s["skipped"] == 1 and s["last_change"] == 0.0
    rel = dit.rel_l2(v2, v1)
    log(f"  repeated step skipped: vel rel_l2 vs the full step {rel:.2e}")
    assert rel < 1e-5
    # reset empties the cache: the next step runs every block again
    fbc.reset()
    _fbc_step(g, cache, fbc, t, 0.08)
    s = fbc.stats()
    assert s["steps"] == 1 and s["skipped"] == 0


def _oracle_changes(wl, sw, blocks, ocache, ic, is_, ts, sig, steps):
    """The oracle's change values along its own loop with threshold 0."""
    st = dit.fbc_new_state()
    x = qs.img_tokens(wl, seed=70)
    changes = []
    for k in range(steps):
        v = dit.first_block_cache_step(sw, blocks, x, ts[k], ic, is_, wl.heads, ocache, st, 0.0)
        changes.append(st["last_change"])
        x = dit.euler_update(x, v.astype(np.float32), sig[k], sig[k + 1])
    return changes


@pytest.mark.parametrize("wl_id,n_blocks", [(1, 3), (2, 2)])
def test_fbc_loop_matches_oracle(wl_id, n_blocks):
    import torch
    wl, g, cache, fbc = _setup(wl_id, n_blocks)
    steps = 6
    sig, tsteps = qi.flow_sigmas(steps, wl.N)
    ts = [np.float32(tsteps[k]) / np.float32(1000) for k in range(steps)]
    sw = qs.weights_as_f32(qs.shared_weights(wl))
    blocks = [qs.weights_as_f32(qs.block_weights(wl, b)) for b in range(wl.n_blocks)]
    tc, tsn, ic, is_ = dit.rope_rows(wl.L, wl.h, wl.w)
    _, ocache = dit.dit_step(sw, blocks, wl.L, qs.img_tokens(wl), qs.txt_feats(wl), np.float32(0.95), tc, tsn,
                             ic, is_, wl.heads, capture=True)
    changes = _oracle_changes(wl, sw, blocks, ocache, ic, is_, ts, sig, steps)
    finite = sorted(c for c in changes if math.isfinite(c))
    log(f"  oracle changes (threshold 0): {['%.4g' % c for c in changes]}")
    thresholds = [0.5 * finite[0], 2.0 * finite[-1]]
    for lo, hi in zip(finite, finite[1:]):
        if hi > 1.5 * lo:
            thresholds.append(math.sqrt(lo * hi))
            break
    for thr in thresholds:
        fbc.reset()
        st = dit.fbc_new_state()
        x = torch.from_numpy(qs.img_tokens(wl, seed=70)).cuda()
        got_skips, ref_skips = [], []
        for k in range(steps):
            x_np = host(x).copy()
            before = st["skipped"]
            ref = dit.first_block_cache_step(sw, blocks, x_np, ts[k], ic, is_, wl.heads, ocache, st, thr)
            ref_skips.append(st["skipped"] - before)
            before = fbc.stats()["skipped"]
            qi.dit_step_fbc(g.model, g.L, g.N, x, ts[k], g.rope[2], g.rope[3], cache, thr, fbc, g.vel, g.ws)
            s = fbc.stats()
            got_skips.append(s["skipped"] - before)
            v = host(g.vel).copy()
            rel, corr = dit.rel_l2(v, ref), dit.min_token_corr(v, ref)
            log(f"  thr {thr:.4g} step {k}: skip gpu {got_skips[-1]} oracle {ref_skips[-1]}; change gpu "
                f"{s['last_change']:.4g} oracle {st['last_change']:.4g}; vel rel_l2 {rel:.2e} corr {corr:.6f}")
            assert np.all(np.isfinite(v)) and rel <= REL_L2_BAR and corr >= CORR_BAR
            qi.euler_update(x, g.vel, sig[k], sig[k + 1])
        assert got_skips == ref_skips, (thr, got_skips, ref_skips)
