"""Helpers shared by the GPU tests: upload a seeded workload, run the HIP path
through the C ABI, and bring results back to the host.  Oracle results are
computed by the tests themselves from the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import block_causal_attention_qi_amd as qi
import qi_synth as qs


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dims_of(wl) -> "qi.QiDims":
    return qi.make_dims(wl.hidden, wl.ffn, wl.n_blocks, wl.txt_dim)


class GpuWorkload:
    """A workload's weights on the device, its inputs and the RoPE rows the
    library computes."""

    def __init__(self, wl, n_blocks=None, device="cuda", threads=8):
        import torch
        self.wl = wl
        nb = wl.n_blocks if n_blocks is None else n_blocks
        self.dims = qi.make_dims(wl.hidden, wl.ffn, nb, wl.txt_dim)
        self.shared_np = qs.shared_weights(wl, as_bf16=True, threads=threads)
        blocks = (qs.block_weights(wl, b, as_bf16=True, threads=threads) for b in range(nb))
        self.model = qi.DeviceModel(self.dims, self.shared_np, blocks, device)
        self.L, self.N = wl.L, wl.N
        self.device = device
        self.set_inputs(qs.img_tokens(wl), qs.txt_feats(wl))
        tc, ts, ic, is_ = qi.rope_tables(wl.L, wl.h, wl.w)
        self.rope_np = (tc, ts, ic, is_)
        self.rope = [torch.from_numpy(a).to(device) for a in (tc, ts, ic, is_)]
        self.ws = qi.Workspace(self.dims, wl.L, wl.N, device)
        self.vel = torch.empty((wl.N, 64), dtype=torch.float32, device=device)

    def set_inputs(self, img_tokens: np.ndarray, txt_feats: np.ndarray | None):
        import torch
        self.img_np = img_tokens
        self.img = torch.from_numpy(np.ascontiguousarray(img_tokens)).to(self.device)
        if txt_feats is not None:
            self.txt_np = txt_feats
            self.txt = torch.from_numpy(np.ascontiguousarray(txt_feats)).to(self.device)

    def new_cache(self):
        return qi.KVCache(self.dims, self.L, self.device)

    def step(self, t, cache=None, vel=None):
        vel = self.vel if vel is None else vel
        tc, ts, ic, is_ = self.rope
        qi.dit_step(self.model, self.L, self.N, self.img, self.txt, t, tc, ts, ic, is_, vel, self.ws, cache)
        return vel

    def capture(self, t, cache, vel=None):
        vel = self.vel if vel is None else vel
        tc, ts, ic, is_ = self.rope
        qi.text_kv_capture(self.model, self.L, self.N, self.img, self.txt, t, tc, ts, ic, is_, cache, vel,
                           self.ws)
        return vel


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str = ""):
    """Bit-for-bit equality of two arrays, reported as a count and the first
    mismatching index (never as a diff of the raw bytes)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, (what, a.shape, b.shape, a.dtype, b.dtype)
    ua = a.reshape(-1).view(np.uint8)
    ub = b.reshape(-1).view(np.uint8)
    bad = np.flatnonzero(ua != ub)
    assert bad.size == 0, f"{what}: {bad.size} differing bytes of {ua.size}, first at byte {bad[0]}"


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bf16_bits(a: np.ndarray) -> np.ndarray:
    return qs.f32_to_bf16_bits(a.astype(np.float32))


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return qs.bf16_bits_to_f32(bits).astype(np.float64)


def unpack_cache_block(cache_np: np.ndarray, dims, L: int, b: int):
    """Split block b's cache slot (int16 bits) into K [heads, L, 128] and V
    [heads, L, 128] as float64 values."""
    heads = dims.heads
    Lp = (L + 63) // 64 * 64
    slot = heads * 128 * (L + Lp)
    s = cache_np[b * slot:(b + 1) * slot].view(np.uint16)
    k = bf16_vals(s[:heads * L * 128]).reshape(heads, L, 128)
    vt = bf16_vals(s[heads * L * 128:]).reshape(heads, 128, Lp)[:, :, :L]
    return k, np.ascontiguousarray(vt.transpose(0, 2, 1))
