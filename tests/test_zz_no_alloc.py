"""The allocation-free step (qi_dit_step_noalloc) against qi_dit_step with a
caller workspace: the same kernels, so bit-identical vel, on consecutive
calls that share the library's static scratch -- a full-width block at
L 22 / N 256, then a smaller request (L 9, N 64), then an image-only step on
a captured cache, then the first request again -- and a request larger than
the scratch is refused on the host before anything is enqueued."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from block_causal_attention_qi_amd import _lib
from tests.gpu_util import assert_bits_equal, host, log

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class _Req:
    def __init__(self, model, dims, wl):
        import torch
        self.model, self.dims, self.wl = model, dims, wl
        self.img, self.txt = _dev(qs.img_tokens(wl)), _dev(qs.txt_feats(wl))
        self.rope = [_dev(a) for a in qi.rope_tables(wl.L, wl.h, wl.w)]
        self.ws = qi.Workspace(dims, wl.L, wl.N)
        self.vel = torch.empty((wl.N, 64), dtype=torch.float32, device="cuda")
        self.t = np.float32(0.7)

    def step(self, noalloc, cache=None):
        tc, ts, ic, is_ = self.rope
        txt, tc, ts = (None, None, None) if cache is not None else (self.txt, tc, ts)
        self.vel.fill_(float("nan"))
        if noalloc:
            qi.dit_step_noalloc(self.model, self.wl.L, self.wl.N, self.img, txt, self.t, tc, ts, ic, is_, self.vel,
                                cache)
        else:
            qi.dit_step(self.model, self.wl.L, self.wl.N, self.img, txt, self.t, tc, ts, ic, is_, self.vel, self.ws,
                        cache)
        return host(self.vel).copy()


def test_noalloc_step_matches_the_workspace_step_on_consecutive_calls():
    wl2 = qs.workload(2)
    dims = qi.make_dims(wl2.hidden, wl2.ffn, wl2.n_blocks, wl2.txt_dim)
    model = qi.DeviceModel(dims, qs.shared_weights(wl2, as_bf16=True),
                           [qs.block_weights(wl2, 0, as_bf16=True)])
    big = _Req(model, dims, wl2)
    small = _Req(model, dims, qs.workload(2, L=9, h=8, w=8))
    assert qi.workspace_bytes(dims, 22, 256) <= _lib.QI_NOALLOC_SCRATCH_BYTES
    for i, r in enumerate((big, small, big)):
        log(f"call {i}: L={r.wl.L} N={r.wl.N}")
        got = r.step(True)
        assert np.all(np.isfinite(got))
        assert_bits_equal(got, r.step(False), f"call {i}: noalloc vs workspace step")
    # image-only on a captured cache, through the scratch
    cache = qi.KVCache(dims, small.wl.L)
    tc, ts, ic, is_ = small.rope
    qi.text_kv_capture(model, small.wl.L, small.wl.N, small.img, small.txt, small.t, tc, ts, ic, is_, cache,
                       small.vel, small.ws)
    full = host(small.vel).copy()
    got = small.step(True, cache)
    assert_bits_equal(got, small.step(False, cache), "image-only: noalloc vs workspace step")
    assert_bits_equal(got, full, "image-only noalloc vs joint")


def test_noalloc_refuses_requests_beyond_the_scratch():
    """The 1024^2 request needs more than the scratch: refused with
    QI_ERR_WORKSPACE on the host (the size check precedes every other use of
    the arguments, so the placeholder pointers here are never read)."""
    wl = qs.workload(4)
    dims = qi.make_dims(wl.hidden, wl.ffn, wl.n_blocks, wl.txt_dim)
    assert qi.workspace_bytes(dims, wl.L, wl.N) > _lib.QI_NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    import ctypes
    st = lib.qi_dit_step_noalloc(ctypes.byref(dims), None, wl.L, wl.N, None, None, 0.5, None, None, None, None,
                                 None, None, None)
    assert st == _lib.QI_ERR_WORKSPACE
