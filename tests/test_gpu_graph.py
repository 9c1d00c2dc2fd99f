"""HIP-graph replay of a denoising-loop step.

The library launches nothing but kernels on the caller's stream (no
allocation, copy, memset or synchronisation inside qi_dit_step or
qi_euler_update), so a caller may capture a step into a graph and replay it.
A captured image-only step (cached text K/V) plus its Euler update must give
the same bits as the same step run eagerly, on every replay: each replay here
starts from a latent reset by an eager copy and a velocity buffer cleared by
an eager fill, with synchronisations between replays."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from tests.gpu_util import GpuWorkload, assert_bits_equal, host, log

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.mark.parametrize("wl_id", [1, 2])
def test_graph_replay_equals_eager_step(wl_id):
    import torch
    wl = qs.workload(wl_id)
    log(f"graph replay: {wl.name}")
    g = GpuWorkload(wl)
    L, N = g.L, g.N
    tc, ts, ic, is_ = g.rope
    sig, tsteps = qi.flow_sigmas(8, N)
    tin = [np.float32(tsteps[i]) / np.float32(1000) for i in range(8)]
    cache = g.new_cache()
    x = g.img.clone()
    vel = g.vel
    qi.text_kv_capture(g.model, L, N, x, g.txt, tin[0], tc, ts, ic, is_, cache, vel, g.ws)
    qi.euler_update(x, vel, sig[0], sig[1])
    x1 = x.clone()

    def step():
        qi.dit_step(g.model, L, N, x, None, tin[1], None, None, ic, is_, vel, g.ws, cache)
        qi.euler_update(x, vel, sig[1], sig[2])

    step()  # eager reference
    torch.cuda.synchronize()
    ref_x, ref_v = host(x).copy(), host(vel).copy()
    assert np.all(np.isfinite(ref_x))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        x.copy_(x1)
        vel.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(host(x), ref_x, f"latent after replay {r}")
        assert_bits_equal(host(vel), ref_v, f"velocity after replay {r}")
