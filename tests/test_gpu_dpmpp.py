"""GPU parity of the DPM++ 2M update (reading S22; the sampler [MLX]
"Optional modes" names): the fused fp32 kernel equals the oracle's fp32 step
bit for bit on random inputs at the first, second-order, middle and final
steps of the 40-step schedule, x and the carried data prediction alike; and a
6-step DPM++ loop of the reduced DiT, each GPU update equal to the oracle's
update of the same latents and vel, the final latent within the parity bar
of the oracle's own loop."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import GpuWorkload, assert_bits_equal, host, log

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("n", [64 * 4096, 1001])
def test_dpmpp_kernel_bit_exact(n):
    rng = np.random.default_rng(n)
    sig, _ = qi.flow_sigmas(40, 4096)
    for i in (0, 1, 2, 20, 39):
        x, v, xp = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
        prev = None if i == 0 else sig[i - 1]
        xd, vd, xpd = _dev(x), _dev(v), _dev(xp)
        qi.dpmpp_2m_update(xd, vd, xpd, prev, sig[i], sig[i + 1])
        want_x, want_x0 = dit.dpmpp_2m_step(x, v, xp, prev, sig[i], sig[i + 1])
        assert_bits_equal(host(xd), want_x, f"x, step {i}")
        assert_bits_equal(host(xpd), want_x0, f"x0, step {i}")


def test_dpmpp_loop_on_the_dit():
    import torch
    wl = qs.workload(1)
    g = GpuWorkload(wl)
    steps = 6
    sig, tsteps = qi.flow_sigmas(steps, wl.N)
    ts = [np.float32(tsteps[k]) / np.float32(1000) for k in range(steps)]
    cache = g.new_cache()
    x = torch.from_numpy(qs.img_tokens(wl)).cuda()
    x0p = torch.zeros_like(x)
    g.set_inputs(qs.img_tokens(wl), None)
    tc, tsn, ic, is_ = g.rope
    for k in range(steps):
        if k == 0:
            qi.text_kv_capture(g.model, wl.L, wl.N, x, g.txt, ts[k], tc, tsn, ic, is_, cache, g.vel, g.ws)
        else:
            qi.dit_step(g.model, wl.L, wl.N, x, None, ts[k], None, None, ic, is_, g.vel, g.ws, cache)
        xh, vh, ph = host(x).copy(), host(g.vel).copy(), host(x0p).copy()
        prev = None if k == 0 else sig[k - 1]
        qi.dpmpp_2m_update(x, g.vel, x0p, prev, sig[k], sig[k + 1])
        want_x, want_x0 = dit.dpmpp_2m_step(xh, vh, ph, prev, sig[k], sig[k + 1])
        assert_bits_equal(host(x), want_x, f"loop x, step {k}")
        assert_bits_equal(host(x0p), want_x0, f"loop x0, step {k}")
    # the oracle's own loop (its own vel) ends close by
    sw = qs.weights_as_f32(qs.shared_weights(wl))
    blocks = [qs.weights_as_f32(qs.block_weights(wl, b)) for b in range(wl.n_blocks)]
    otc, ots, oic, ois = dit.rope_rows(wl.L, wl.h, wl.w)
    xo = qs.img_tokens(wl)
    ref_x0p = np.zeros_like(xo)
    _, ocache = dit.dit_step(sw, blocks, wl.L, xo, qs.txt_feats(wl), ts[0], otc, ots, oic, ois, wl.heads, capture=True)
    for k in range(steps):
        v = dit.dit_step(sw, blocks, wl.L, xo, None, ts[k], None, None, oic, ois, wl.heads, kv_cache=ocache)
        xo, ref_x0p = dit.dpmpp_2m_step(xo, v.astype(np.float32), ref_x0p, None if k == 0 else sig[k - 1], sig[k],
                                        sig[k + 1])
    rel = dit.rel_l2(host(x), xo)
    log(f"  DPM++ 2M 6-step loop: final latent rel_l2 vs the oracle's loop {rel:.2e}")
    assert rel <= 2e-2
