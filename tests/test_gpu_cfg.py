"""GPU parity of true classifier-free guidance with two K/V slots ([MLX]
"Optional modes": noise = neg + g * (pos - neg), a second forward per step;
"Text K/V reuse": the negative prompt's K/V in a second slot, and a CFG
render with reuse matching full recomputation to the last pixel):

  - the fused CFG Euler update equals the oracle's bit for bit (the float4
    path and the scalar tail path);
  - a CFG image-only step (both branches through every block at once, 2N
    rows) gives, per branch, exactly the vel of qi_dit_step on that branch's
    cache alone and of that branch's full joint recompute;
  - each branch and the guided prediction against the oracle (each branch an
    oracle step on its own prompt, combined as the page writes it).

Workloads: the reduced block (hidden 512, L 8 / negative 4, N 64), a ragged
2-block variant (L 37 / 18, 9x7) and the full-width block (hidden 4096, L 22
/ 11, N 256).  The negative prompt is the seeded stand-in of qi_synth."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import GpuWorkload, assert_bits_equal, host, log

pytestmark = pytest.mark.gpu

REL_L2_BAR = 2e-2
CORR_BAR = 0.999
GUIDANCE = 2.5   # the --cfg value the MLX page's option table shows


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Cfg:
    """A workload with a positive (the workload's) and a negative prompt."""

    def __init__(self, wl):
        import torch
        self.g = g = GpuWorkload(wl)
        self.wl, self.N, self.Lp = wl, wl.N, wl.L
        self.Ln = qs.neg_prompt_len(wl)
        self.txt_neg_np = qs.neg_txt_feats(wl)
        self.txt_neg = _dev(self.txt_neg_np)
        self.rope_neg_np = qi.rope_tables(self.Ln, wl.h, wl.w)
        self.rope_neg = [_dev(a) for a in self.rope_neg_np]
        self.ws_neg = qi.Workspace(g.dims, self.Ln, self.N)
        self.cache_pos = qi.KVCache(g.dims, self.Lp)
        self.cache_neg = qi.KVCache(g.dims, self.Ln)
        self.img_cos2 = torch.cat([g.rope[2], self.rope_neg[2]]).contiguous()
        self.img_sin2 = torch.cat([g.rope[3], self.rope_neg[3]]).contiguous()
        self.cws = qi.CfgWorkspace(g.dims, self.N)
        self.vel2 = torch.empty((2, self.N, 64), dtype=torch.float32, device="cuda")
        self.vel_n = torch.empty((self.N, 64), dtype=torch.float32, device="cuda")

    def capture(self, t):
        g = self.g
        g.capture(t, self.cache_pos)
        qi.text_kv_capture(g.model, self.Ln, self.N, g.img, self.txt_neg, t, *self.rope_neg, self.cache_neg,
                           self.vel_n, self.ws_neg)

    def cfg_step(self, t):
        qi.dit_step_cfg(self.g.model, self.N, self.g.img, t, self.img_cos2, self.img_sin2, self.cache_pos,
                        self.cache_neg, self.vel2, self.cws)
        return host(self.vel2).copy()

    def neg_step(self, t, cached: bool):
        g = self.g
        tc, ts, ic, is_ = self.rope_neg
        qi.dit_step(g.model, self.Ln, self.N, g.img, None if cached else self.txt_neg, t, None if cached else tc,
                    None if cached else ts, ic, is_, self.vel_n, self.ws_neg, self.cache_neg if cached else None)
        return host(self.vel_n).copy()


@pytest.mark.parametrize("n", [64 * 256, 1001])
def test_cfg_euler_bit_exact(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32)
    pos = rng.standard_normal(n).astype(np.float32)
    neg = (pos + 0.25 * rng.standard_normal(n)).astype(np.float32)
    sc, sn = np.float32(0.8333), np.float32(0.8125)
    for gd in (GUIDANCE, 0.0, 1.0, -0.75):
        xd = _dev(x)
        vel2 = _dev(np.concatenate([pos, neg]))
        qi.euler_update_cfg(xd, vel2, gd, sc, sn)
        assert_bits_equal(host(xd), dit.euler_update_cfg(x, pos, neg, gd, sc, sn), f"cfg euler g={gd} n={n}")
    # guidance must be finite; nothing is launched otherwise
    with pytest.raises(qi.QiError):
        qi.euler_update_cfg(_dev(x), _dev(np.concatenate([pos, neg])), float("nan"), sc, sn)


@pytest.mark.parametrize("wl_id,over", [(1, {}), (1, dict(L=37, h=9, w=7, n_blocks=2)), (2, {})])
def test_cfg_step_branches_bit_equal_single_and_full(wl_id, over):
    wl = qs.workload(wl_id, **over)
    c = Cfg(wl)
    log(f"cfg wl={wl_id} {over}: L_pos={c.Lp} L_neg={c.Ln} N={c.N} blocks={wl.n_blocks}")
    c.capture(np.float32(0.9))
    assert c.cache_pos.valid and c.cache_neg.valid
    c.g.set_inputs(qs.img_tokens(wl, seed=77), None)
    t2 = np.float32(0.41)
    vel2 = c.cfg_step(t2)
    assert np.all(np.isfinite(vel2))
    pos_cached = host(c.g.step(t2, cache=c.cache_pos)).copy()
    pos_full = host(c.g.step(t2)).copy()
    neg_cached = c.neg_step(t2, cached=True)
    neg_full = c.neg_step(t2, cached=False)
    assert_bits_equal(vel2[0], pos_cached, "CFG pos branch vs single cached step")
    assert_bits_equal(vel2[1], neg_cached, "CFG neg branch vs single cached step")
    assert_bits_equal(vel2[0], pos_full, "CFG pos branch vs full joint recompute")
    assert_bits_equal(vel2[1], neg_full, "CFG neg branch vs full joint recompute")
    assert not np.array_equal(vel2[0], vel2[1])   # the prompts do differ
    # the step is reproducible
    assert_bits_equal(c.cfg_step(t2), vel2, "CFG step rerun")


def _check_bar(v, ref, what):
    rel, corr = dit.rel_l2(v, ref), dit.min_token_corr(v, ref)
    log(f"  {what}: rel_l2={rel:.3e} min_token_corr={corr:.6f}")
    assert np.all(np.isfinite(v)) and rel <= REL_L2_BAR and corr >= CORR_BAR, (what, rel, corr)


@pytest.mark.parametrize("wl_id", [1, 2])
def test_cfg_step_matches_oracle(wl_id):
    import torch
    wl = qs.workload(wl_id)
    c = Cfg(wl)
    t = np.float32(wl.timestep)
    c.capture(t)
    vel2 = c.cfg_step(t)
    # guided prediction on the GPU: the fused update from x = 0 with
    # sigma 0 -> 1 leaves x = 1 * noise = noise exactly
    x = torch.zeros((c.N, 64), dtype=torch.float32, device="cuda")
    qi.euler_update_cfg(x, c.vel2, GUIDANCE, 0.0, 1.0)
    noise = host(x)
    sw = qs.weights_as_f32(qs.shared_weights(wl))
    blocks = [qs.weights_as_f32(qs.block_weights(wl, b)) for b in range(wl.n_blocks)]
    tc, ts, ic, is_ = dit.rope_rows(wl.L, wl.h, wl.w)
    ref_pos = dit.dit_step(sw, blocks, wl.L, qs.img_tokens(wl), qs.txt_feats(wl), t, tc, ts, ic, is_, wl.heads)
    tcn, tsn, icn, isn = dit.rope_rows(c.Ln, wl.h, wl.w)
    ref_neg = dit.dit_step(sw, blocks, c.Ln, qs.img_tokens(wl), c.txt_neg_np, t, tcn, tsn, icn, isn, wl.heads)
    _check_bar(vel2[0], ref_pos, "pos branch")
    _check_bar(vel2[1], ref_neg, "neg branch")
    ref_noise = dit.cfg_combine(ref_pos.astype(np.float32), ref_neg.astype(np.float32), GUIDANCE)
    _check_bar(noise, ref_noise, f"guided prediction g={GUIDANCE}")
    # and the GPU's own combination is the oracle's formula on the GPU branches
    assert_bits_equal(noise, dit.cfg_combine(vel2[0], vel2[1], GUIDANCE), "guided prediction formula")
