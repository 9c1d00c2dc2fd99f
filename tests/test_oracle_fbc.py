"""Pins of the oracle's first-block cache (Fast mode, reading S21), CPU only.

What fixes them: the special cases the definition reduces to -- threshold 0
never skips, so every step is the ordinary cached step (oracle.dit_step); a
step repeated on identical inputs has zero change, so it is skipped at any
positive threshold and reproduces the full step up to float64 rounding; a
first step (empty cache) is never skipped -- and a planted mistake (dropping
the cached residual of the skipped blocks) fails them."""
import math

import numpy as np

import qi_synth as qs
from oracle import dit
from tests.oracle_plant import planted

WL = qs.workload(1, n_blocks=3)


def _setup():
    sw = qs.weights_as_f32(qs.shared_weights(WL))
    blocks = [qs.weights_as_f32(qs.block_weights(WL, b)) for b in range(WL.n_blocks)]
    tc, ts, ic, is_ = dit.rope_rows(WL.L, WL.h, WL.w)
    _, cache = dit.dit_step(sw, blocks, WL.L, qs.img_tokens(WL), qs.txt_feats(WL), np.float32(0.9), tc, ts, ic,
                            is_, WL.heads, capture=True)
    return sw, blocks, cache, ic, is_


def test_threshold_zero_is_the_exact_cached_step():
    sw, blocks, cache, ic, is_ = _setup()
    st = dit.fbc_new_state()
    for k, t in enumerate((0.8, 0.6, 0.6)):
        img = qs.img_tokens(WL, seed=50 + k)
        got = dit.first_block_cache_step(sw, blocks, img, np.float32(t), ic, is_, WL.heads, cache, st, 0.0)
        ref = dit.dit_step(sw, blocks, WL.L, img, None, np.float32(t), None, None, ic, is_, WL.heads,
                           kv_cache=cache)
        assert np.array_equal(got, ref)
    assert st["steps"] == 3 and st["skipped"] == 0


def test_repeated_step_is_skipped_and_reproduces_the_full_step():
    sw, blocks, cache, ic, is_ = _setup()
    st = dit.fbc_new_state()
    img, t = qs.img_tokens(WL, seed=61), np.float32(0.7)
    v1 = dit.first_block_cache_step(sw, blocks, img, t, ic, is_, WL.heads, cache, st, 0.08)
    assert st["skipped"] == 0 and math.isinf(st["last_change"])     # first step: empty cache
    v2 = dit.first_block_cache_step(sw, blocks, img, t, ic, is_, WL.heads, cache, st, 0.08)
    assert st["skipped"] == 1 and st["last_change"] == 0.0
    assert np.allclose(v2, v1, rtol=1e-12, atol=1e-12)
    # a changed latent changes block 0's residual: the change is positive
    dit.first_block_cache_step(sw, blocks, qs.img_tokens(WL, seed=62), t, ic, is_, WL.heads, cache, st, 0.0)
    assert st["last_change"] > 0.0


def test_dropped_cached_residual_fails_the_pins():
    sw, blocks, cache, ic, is_ = _setup()
    bad = planted(dit.first_block_cache_step, "x = x1 + state[\"rem\"]", "x = x1")
    st = dit.fbc_new_state()
    img, t = qs.img_tokens(WL, seed=61), np.float32(0.7)
    v1 = bad(sw, blocks, img, t, ic, is_, WL.heads, cache, st, 0.08)
    v2 = bad(sw, blocks, img, t, ic, is_, WL.heads, cache, st, 0.08)
    assert st["skipped"] == 1 and not np.allclose(v2, v1, rtol=1e-6, atol=1e-6)
