"""Properties at the full sizes, in the launch configuration the benchmark
times (the oracle parity of these workloads, block by block and whole-step,
is in test_gpu_fulldepth.py).

  - 384^2 (hidden 4096, L 494, N 576): a 2-block stack at this shape against
    the exact oracle at the 2e-2 / 0.999 bar.
  - 384^2, 1024^2 (L 407, N 4096) and 2048^2 (L 512, N 16384), all 32
    blocks: the cached image-only step equals the GPU's full recompute bit for
    bit, captured text K/V do not depend on the image tokens or t, no NaN/Inf.
  - 1024^2: true CFG's two branches through every block at once, each equal
    to its single-branch cached step bit for bit.

The 32-block workloads share one set of weights (same widths, depth and
seeds), the session fixture `model32` of conftest.py."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import assert_bits_equal, host, log, unpack_cache_block

pytestmark = pytest.mark.gpu

REL_L2_BAR = 2e-2
CORR_BAR = 0.999


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Run:
    """Inputs, RoPE rows and buffers of one workload on the shared model."""

    def __init__(self, m, wl, img_seed=qs.NOISE_SEED):
        import torch
        self.m, self.wl = m, wl
        self.img = _dev(qs.img_tokens(wl, seed=img_seed))
        self.txt = _dev(qs.txt_feats(wl))
        self.rope = [_dev(a) for a in qi.rope_tables(wl.L, wl.h, wl.w)]
        self.ws = qi.Workspace(m["dims"], wl.L, wl.N)
        self.vel = torch.empty((wl.N, 64), dtype=torch.float32, device="cuda")

    def step(self, t, cache=None):
        tc, ts, ic, is_ = self.rope
        qi.dit_step(self.m["model"], self.wl.L, self.wl.N, self.img, None if cache else self.txt, t,
                    None if cache else tc, None if cache else ts, ic, is_, self.vel, self.ws, cache)
        return host(self.vel).copy()

    def capture(self, t, cache):
        tc, ts, ic, is_ = self.rope
        qi.text_kv_capture(self.m["model"], self.wl.L, self.wl.N, self.img, self.txt, t, tc, ts, ic, is_, cache,
                           self.vel, self.ws)
        return host(self.vel).copy()


def _reuse_properties(m, wl):
    log(f"reuse properties {wl.name}")
    r = Run(m, wl)
    cache = qi.KVCache(m["dims"], wl.L)
    _, ts = qi.flow_sigmas(40, wl.N)
    t0, t1 = np.float32(ts[0]) / np.float32(1000), np.float32(ts[20]) / np.float32(1000)
    v0 = r.capture(t0, cache)
    assert np.all(np.isfinite(v0))
    kv_a = host(cache.buf).copy()
    full = r.step(t1)
    cached = r.step(t1, cache)
    assert np.all(np.isfinite(cached))
    assert_bits_equal(cached, full, "cached vs full recompute")
    log("  cached == full")
    # the text K/V of a capture with other image tokens and another t
    r2 = Run(m, wl, img_seed=4321)
    c2 = qi.KVCache(m["dims"], wl.L)
    r2.capture(t1, c2)
    kv_b = host(c2.buf)
    for b in (0, 15, 31):
        ka, va = unpack_cache_block(kv_a, m["dims"], wl.L, b)
        kb, vb = unpack_cache_block(kv_b, m["dims"], wl.L, b)
        assert_bits_equal(ka, kb, f"K block {b}")
        assert_bits_equal(va, vb, f"V block {b}")
    log("  text K/V invariant")


@pytest.mark.timeout(900)
def test_two_blocks_at_384px_match_oracle(model32):
    """The first two blocks as a 2-block model at the 384^2 shape (L 494,
    N 576), against the exact oracle at the 2e-2 / 0.999 bar."""
    wl = qs.workload(3, n_blocks=2)
    dims = qi.make_dims(wl.hidden, wl.ffn, 2, wl.txt_dim)
    m2 = {"dims": dims, "model": qi.DeviceModel(dims, model32["shared"], model32["blocks"][:2]),
          "blocks": model32["blocks"][:2], "shared": model32["shared"]}
    r = Run(m2, wl)
    t = np.float32(0.7)
    vel = r.step(t)
    sw = qs.weights_as_f32(model32["shared"])
    tc, tsn, ic, is_ = dit.rope_rows(wl.L, wl.h, wl.w)
    ref = dit.dit_step(sw, [qs.weights_as_f32(b) for b in m2["blocks"]], wl.L, qs.img_tokens(wl),
                       qs.txt_feats(wl), t, tc, tsn, ic, is_, wl.heads)
    rel, corr = dit.rel_l2(vel, ref), dit.min_token_corr(vel, ref)
    log(f"  384px 2 blocks: vel rel_l2={rel:.3e} min_token_corr={corr:.6f}")
    assert np.all(np.isfinite(vel)) and rel <= REL_L2_BAR and corr >= CORR_BAR


@pytest.mark.timeout(900)
def test_dit32_384px_reuse_exact(model32):
    _reuse_properties(model32, qs.workload(3))


@pytest.mark.timeout(900)
def test_dit32_1024px_reuse_exact(model32):
    _reuse_properties(model32, qs.workload(4))


@pytest.mark.timeout(900)
def test_dit32_2048px_reuse_exact(model32):
    _reuse_properties(model32, qs.workload(5))


@pytest.mark.timeout(900)
def test_dit32_1024px_cfg_branches_exact(model32):
    """True CFG at 1024^2 with 32 blocks: both branches through every block at
    once (8192 image rows), each branch bit-equal to the single-branch cached
    step on its own K/V slot (L 407 and the 203-token negative prompt)."""
    import torch
    wl = qs.workload(4)
    r = Run(model32, wl)
    Ln = qs.neg_prompt_len(wl)
    log(f"cfg at {wl.name}: L_pos={wl.L} L_neg={Ln}")
    txt_neg = _dev(qs.neg_txt_feats(wl))
    rope_n = [_dev(a) for a in qi.rope_tables(Ln, wl.h, wl.w)]
    ws_n = qi.Workspace(model32["dims"], Ln, wl.N)
    c_pos, c_neg = qi.KVCache(model32["dims"], wl.L), qi.KVCache(model32["dims"], Ln)
    vel_n = torch.empty((wl.N, 64), dtype=torch.float32, device="cuda")
    _, ts = qi.flow_sigmas(40, wl.N)
    t0, t1 = np.float32(ts[0]) / np.float32(1000), np.float32(ts[20]) / np.float32(1000)
    r.capture(t0, c_pos)
    qi.text_kv_capture(model32["model"], Ln, wl.N, r.img, txt_neg, t0, *rope_n, c_neg, vel_n, ws_n)
    cws = qi.CfgWorkspace(model32["dims"], wl.N)
    vel2 = torch.empty((2, wl.N, 64), dtype=torch.float32, device="cuda")
    cos2 = torch.cat([r.rope[2], rope_n[2]]).contiguous()
    sin2 = torch.cat([r.rope[3], rope_n[3]]).contiguous()
    qi.dit_step_cfg(model32["model"], wl.N, r.img, t1, cos2, sin2, c_pos, c_neg, vel2, cws)
    got = host(vel2).copy()
    assert np.all(np.isfinite(got))
    assert_bits_equal(got[0], r.step(t1, c_pos), "CFG pos branch vs single cached step")
    qi.dit_step(model32["model"], Ln, wl.N, r.img, None, t1, None, None, rope_n[2], rope_n[3], vel_n, ws_n, c_neg)
    assert_bits_equal(got[1], host(vel_n), "CFG neg branch vs single cached step")
    log("  both branches bit-equal")
