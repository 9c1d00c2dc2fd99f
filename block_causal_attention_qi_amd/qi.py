"""Python binding of libqi (include/qi.h): argument marshalling only.

Every step of the DiT runs in the HIP library.  torch provides device memory
(tensors whose data pointers are handed to the C ABI) and the stream; numpy
arrays carry the host-side tables.  bf16 weights travel as uint16 bit
patterns and are stored on the device as int16 tensors of the same bits."""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (QI_MODE_IMAGE_ONLY, QI_MODE_JOINT, QiBlockW, QiDims, QiEncDims, QiEncLayerW, QiEncModelW,
                   QiError, QiKvCache, QiModelW, check)

__all__ = ["QI_MODE_JOINT", "QI_MODE_IMAGE_ONLY", "QiError", "make_dims", "rope_axis_table",
           "rope_tables", "flow_sigmas", "workspace_bytes", "kv_cache_bytes", "kv_slot_elems",
           "DeviceModel", "KVCache", "Workspace", "dit_step", "dit_step_noalloc", "text_kv_capture", "dit_block_fwd",
           "euler_update", "modulation", "block_causal_attention", "linear_bf16", "stream_handle",
           "timing_begin", "timing_end", "KERNEL_KINDS", "cfg_workspace_bytes", "CfgWorkspace", "dit_step_cfg",
           "euler_update_cfg", "fbc_bytes", "FirstBlockCache", "dit_step_fbc", "dpmpp_2m_coeffs",
           "dpmpp_2m_update", "make_enc_dims", "enc_rope_table", "enc_workspace_bytes", "DeviceEncoder",
           "EncWorkspace", "text_encoder_fwd"]


def _np_ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _ptr(t) -> int:
    """Device pointer of a torch tensor (0 for None)."""
    if t is None:
        return 0
    return int(t.data_ptr())


def stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def make_dims(hidden: int, ffn: int, n_blocks: int, txt_dim: int) -> QiDims:
    return QiDims(hidden, hidden // 128, 128, ffn, n_blocks, txt_dim)


# ------------------------------------------------------------------ host tables

def rope_axis_table(d: int):
    lib = _lib.load()
    c = np.empty((9216, d // 2), np.float32)
    s = np.empty_like(c)
    check(lib.qi_rope_axis_table(d, _np_ptr(c), _np_ptr(s)), "qi_rope_axis_table")
    return c, s


def rope_tables(L: int, h: int, w: int):
    """(txt_cos, txt_sin, img_cos, img_sin) host fp32 arrays [L,64], [L,64],
    [h*w,64], [h*w,64]."""
    lib = _lib.load()
    tc = np.empty((max(L, 1), 64), np.float32)
    ts = np.empty_like(tc)
    ic = np.empty((h * w, 64), np.float32)
    is_ = np.empty_like(ic)
    check(lib.qi_rope_tables(L, h, w, _np_ptr(tc), _np_ptr(ts), _np_ptr(ic), _np_ptr(is_)), "qi_rope_tables")
    return tc[:L], ts[:L], ic, is_


def flow_sigmas(steps: int, n_img_tokens: int):
    lib = _lib.load()
    s = np.empty(steps + 1, np.float32)
    t = np.empty(steps, np.float32)
    check(lib.qi_flow_sigmas(steps, n_img_tokens, _np_ptr(s), _np_ptr(t)), "qi_flow_sigmas")
    return s, t


def workspace_bytes(dims: QiDims, L: int, N: int) -> int:
    return int(_lib.load().qi_workspace_bytes(ctypes.byref(dims), L, N))


def kv_cache_bytes(dims: QiDims, L: int) -> int:
    return int(_lib.load().qi_kv_cache_bytes(ctypes.byref(dims), L))


def kv_slot_elems(dims: QiDims, L: int) -> int:
    return int(_lib.load().qi_kv_slot_elems(ctypes.byref(dims), L))


# ------------------------------------------------------------------ device objects

def to_device(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceModel:
    """Device copies of the DiT weights and the C structs that point at them.

    shared: dict of the shared tensors; blocks: sequence (or iterable) of
    per-block dicts.  Linear weights must already be bf16 bit patterns
    (uint16); norms and biases fp32."""

    BLOCK_KEYS = ("w_qkv", "w_o", "w_gu", "w_down", "norm1", "norm2")
    SHARED_KEYS = ("w_mod", "b_mod", "w_img", "b_img", "txt_norm", "w_txt", "b_txt",
                   "norm_out", "w_out", "b_out")

    def __init__(self, dims: QiDims, shared: dict, blocks, device="cuda"):
        self.dims = dims
        self.device = device
        self.shared = {k: to_device(_as_dev(k, shared[k]), device) for k in self.SHARED_KEYS}
        self.blocks = []
        for bw in blocks:
            self.blocks.append({k: to_device(_as_dev(k, bw[k]), device) for k in self.BLOCK_KEYS})
        if len(self.blocks) != dims.n_blocks:
            raise ValueError(f"{len(self.blocks)} blocks given, dims say {dims.n_blocks}")
        self._bw = (QiBlockW * len(self.blocks))()
        for i, b in enumerate(self.blocks):
            self._bw[i] = QiBlockW(*(_ptr(b[k]) for k in self.BLOCK_KEYS))
        sh = self.shared
        self.w = QiModelW(ctypes.cast(self._bw, ctypes.POINTER(QiBlockW)),
                          *(_ptr(sh[k]) for k in self.SHARED_KEYS))

    def block_struct(self, b: int) -> QiBlockW:
        return self._bw[b]

    def prefix(self, n_blocks: int) -> "DeviceModel":
        """The model made of this one's first n_blocks blocks (all device
        weights shared; a one-block workload of the same width and seeds is
        block 0 of the deeper ones)."""
        if not 1 <= n_blocks <= self.dims.n_blocks:
            raise ValueError(f"n_blocks {n_blocks} outside 1..{self.dims.n_blocks}")
        m = DeviceModel.__new__(DeviceModel)
        d = self.dims
        m.dims = QiDims(d.hidden, d.heads, d.head_dim, d.ffn, n_blocks, d.txt_dim)
        m.device, m.shared, m.blocks, m._bw, m.w = self.device, self.shared, self.blocks[:n_blocks], self._bw, self.w
        return m

    def with_shared(self, shared: dict) -> "DeviceModel":
        """A model that shares this one's device block weights and has its own
        copies of the shared weights (modulation, embed, text projection,
        head)."""
        m = DeviceModel.__new__(DeviceModel)
        m.dims, m.device, m.blocks, m._bw = self.dims, self.device, self.blocks, self._bw
        m.shared = {k: to_device(_as_dev(k, shared[k]), self.device) for k in self.SHARED_KEYS}
        sh = m.shared
        m.w = QiModelW(ctypes.cast(m._bw, ctypes.POINTER(QiBlockW)), *(_ptr(sh[k]) for k in self.SHARED_KEYS))
        return m


def _as_dev(name: str, a: np.ndarray) -> np.ndarray:
    """Linear weights go to the device as bf16 bits; fp32 arrays given for a
    2-D weight are a caller error (the library reads bf16 only)."""
    if a.ndim == 2 and a.dtype != np.uint16:
        raise TypeError(f"{name}: 2-D weights must be bf16 bit patterns (uint16), got {a.dtype}")
    if a.ndim == 1 and a.dtype != np.float32:
        a = a.astype(np.float32)
    return a


class KVCache:
    """Text K/V cache ([blocks][K heads x L x 128 | V^T heads x 128 x Lp] bf16)."""

    def __init__(self, dims: QiDims, L: int, device="cuda"):
        import torch
        self.nbytes = kv_cache_bytes(dims, L)
        # zero-filled so the never-written V^T padding columns hold defined bits
        self.buf = torch.zeros(self.nbytes // 2, dtype=torch.int16, device=device)
        self.c = QiKvCache(_ptr(self.buf), L, dims.n_blocks, dims.hidden, 0)
        self.slot_elems = kv_slot_elems(dims, L)

    @property
    def valid(self) -> bool:
        return bool(self.c.valid)

    def slot_ptr(self, b: int) -> int:
        return _ptr(self.buf) + 2 * b * self.slot_elems


def cfg_workspace_bytes(dims: QiDims, N: int) -> int:
    return int(_lib.load().qi_cfg_workspace_bytes(ctypes.byref(dims), N))


class CfgWorkspace:
    """Workspace of a true-CFG image-only step (both branches)."""

    def __init__(self, dims: QiDims, N: int, device="cuda"):
        import torch
        self.nbytes = cfg_workspace_bytes(dims, N)
        if self.nbytes == 0:
            raise ValueError("invalid dims or N for the CFG workspace")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return _ptr(self.buf)


def fbc_bytes(dims: QiDims, N: int) -> int:
    return int(_lib.load().qi_fbc_bytes(ctypes.byref(dims), N))


class FirstBlockCache:
    """Device buffer of the first-block cache (Fast mode) for N image rows."""

    def __init__(self, dims: QiDims, N: int, device="cuda", stream=None):
        import torch
        self.nbytes = fbc_bytes(dims, N)
        if self.nbytes == 0:
            raise ValueError("invalid dims or N for the first-block cache")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.reset(stream)

    @property
    def ptr(self) -> int:
        return _ptr(self.buf)

    def reset(self, stream=None):
        check(_lib.load().qi_fbc_reset(self.ptr, self.nbytes, stream_handle(stream)), "qi_fbc_reset")

    def stats(self, stream=None) -> dict:
        """{'steps', 'skipped', 'last_change'} (synchronises the stream)."""
        n, k, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
        check(_lib.load().qi_fbc_stats(self.ptr, ctypes.byref(n), ctypes.byref(k), ctypes.byref(c),
                                       stream_handle(stream)), "qi_fbc_stats")
        return {"steps": n.value, "skipped": k.value, "last_change": c.value}


class Workspace:
    def __init__(self, dims: QiDims, L: int, N: int, device="cuda"):
        import torch
        self.nbytes = workspace_bytes(dims, L, N)
        if self.nbytes == 0:
            raise ValueError("invalid dims for the workspace")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return _ptr(self.buf)


# ------------------------------------------------------------------ text encoder

def make_enc_dims(hidden: int, heads: int, kv_heads: int, ffn: int, n_layers: int, vocab: int) -> QiEncDims:
    return QiEncDims(hidden, heads, kv_heads, 128, ffn, n_layers, vocab)


def enc_rope_table(L: int, theta: float = 5.0e6):
    """Host fp32 RoPE rows (cos, sin) [L, 64] of positions 0..L-1."""
    c = np.empty((L, 64), np.float32)
    s = np.empty((L, 64), np.float32)
    check(_lib.load().qi_enc_rope_table(L, float(theta), _np_ptr(c), _np_ptr(s)), "qi_enc_rope_table")
    return c, s


def enc_workspace_bytes(dims: QiEncDims, L: int) -> int:
    return int(_lib.load().qi_enc_workspace_bytes(ctypes.byref(dims), L))


class EncWorkspace:
    def __init__(self, dims: QiEncDims, L: int, device="cuda"):
        import torch
        self.nbytes = enc_workspace_bytes(dims, L)
        if self.nbytes == 0:
            raise ValueError("invalid encoder dims or L")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)

    @property
    def ptr(self) -> int:
        return _ptr(self.buf)


class DeviceEncoder:
    """Device copies of the encoder weights.  layers: iterable of per-layer
    dicts with w_q, w_k, w_v, q_norm, k_norm, w_o, w_gate, w_up, w_down,
    in_norm, post_norm (2-D weights as bf16 bits); embed: [vocab, hidden] bf16
    bits.  q/k/v and gate/up are concatenated into the layouts the library
    reads (w_qkv: q rows, k rows, v rows; w_gu: gate rows, up rows)."""

    def __init__(self, dims: QiEncDims, embed: np.ndarray, layers, device="cuda"):
        self.dims = dims
        self.embed = to_device(_as_dev("embed", embed), device)
        self.layers = []
        for lw in layers:
            d = {
                "w_qkv": np.concatenate([lw["w_q"], lw["w_k"], lw["w_v"]], axis=0),
                "q_norm": lw["q_norm"], "k_norm": lw["k_norm"], "w_o": lw["w_o"],
                "w_gu": np.concatenate([lw["w_gate"], lw["w_up"]], axis=0),
                "w_down": lw["w_down"], "in_norm": lw["in_norm"], "post_norm": lw["post_norm"],
            }
            self.layers.append({k: to_device(_as_dev(k, v), device) for k, v in d.items()})
        if len(self.layers) != dims.n_layers:
            raise ValueError(f"{len(self.layers)} layers given, dims say {dims.n_layers}")
        keys = ("w_qkv", "q_norm", "k_norm", "w_o", "w_gu", "w_down", "in_norm", "post_norm")
        self._lw = (QiEncLayerW * len(self.layers))()
        for i, lw in enumerate(self.layers):
            self._lw[i] = QiEncLayerW(*(_ptr(lw[k]) for k in keys))
        self.w = QiEncModelW(ctypes.cast(self._lw, ctypes.POINTER(QiEncLayerW)), _ptr(self.embed))


def text_encoder_fwd(enc: DeviceEncoder, ids, L: int, cos, sin, hidden, ws: EncWorkspace, stream=None):
    """hidden [L, hidden] (device fp32) <- the encoder on ids [L] (device int32)."""
    st = _lib.load().qi_text_encoder_fwd(ctypes.byref(enc.dims), ctypes.byref(enc.w), _ptr(ids), L, _ptr(cos),
                                         _ptr(sin), _ptr(hidden), ws.ptr, ws.nbytes, stream_handle(stream))
    check(st, "qi_text_encoder_fwd")


# ------------------------------------------------------------------ entry points

def dit_step(model: DeviceModel, L: int, N: int, img_tokens, txt_feats, t: float, txt_cos, txt_sin,
             img_cos, img_sin, vel, ws: Workspace, cache: KVCache | None = None, stream=None):
    lib = _lib.load()
    st = lib.qi_dit_step(ctypes.byref(model.dims), ctypes.byref(model.w), L, N, _ptr(img_tokens),
                         _ptr(txt_feats), float(t), _ptr(txt_cos), _ptr(txt_sin), _ptr(img_cos),
                         _ptr(img_sin), ctypes.byref(cache.c) if cache is not None else None,
                         _ptr(vel), ws.ptr, ws.nbytes, stream_handle(stream))
    check(st, "qi_dit_step")


def dit_step_noalloc(model: DeviceModel, L: int, N: int, img_tokens, txt_feats, t: float, txt_cos, txt_sin,
                     img_cos, img_sin, vel, cache: KVCache | None = None, stream=None):
    """qi_dit_step on the library's static per-GPU scratch (no workspace)."""
    lib = _lib.load()
    st = lib.qi_dit_step_noalloc(ctypes.byref(model.dims), ctypes.byref(model.w), L, N, _ptr(img_tokens),
                                 _ptr(txt_feats), float(t), _ptr(txt_cos), _ptr(txt_sin), _ptr(img_cos),
                                 _ptr(img_sin), ctypes.byref(cache.c) if cache is not None else None,
                                 _ptr(vel), stream_handle(stream))
    check(st, "qi_dit_step_noalloc")


def text_kv_capture(model: DeviceModel, L: int, N: int, img_tokens, txt_feats, t: float, txt_cos,
                    txt_sin, img_cos, img_sin, cache: KVCache, vel, ws: Workspace, stream=None):
    lib = _lib.load()
    st = lib.qi_text_kv_capture(ctypes.byref(model.dims), ctypes.byref(model.w), L, N, _ptr(img_tokens),
                                _ptr(txt_feats), float(t), _ptr(txt_cos), _ptr(txt_sin), _ptr(img_cos),
                                _ptr(img_sin), ctypes.byref(cache.c), _ptr(vel), ws.ptr, ws.nbytes,
                                stream_handle(stream))
    check(st, "qi_text_kv_capture")


def dit_block_fwd(dims: QiDims, block: QiBlockW, L: int, N: int, mode: int, x, mod, cos, sin,
                  kv_slot_ptr: int, ws: Workspace, stream=None):
    lib = _lib.load()
    st = lib.qi_dit_block_fwd(ctypes.byref(dims), ctypes.byref(block), L, N, mode, _ptr(x), _ptr(mod),
                              _ptr(cos), _ptr(sin), kv_slot_ptr or None, ws.ptr, ws.nbytes,
                              stream_handle(stream))
    check(st, "qi_dit_block_fwd")


def euler_update(x, vel, sigma_cur: float, sigma_next: float, stream=None):
    n = x.numel()
    if vel.numel() != n:
        raise ValueError("x and vel sizes differ")
    st = _lib.load().qi_euler_update(_ptr(x), _ptr(vel), float(sigma_cur), float(sigma_next), n,
                                     stream_handle(stream))
    check(st, "qi_euler_update")


def dit_step_cfg(model: DeviceModel, N: int, img_tokens, t: float, img_cos2, img_sin2, cache_pos: KVCache,
                 cache_neg: KVCache, vel2, ws: CfgWorkspace, stream=None):
    """True-CFG image-only step: img_cos2/img_sin2 [2, N, 64] (branch rows),
    vel2 [2, N, 64] out ([pos | neg])."""
    st = _lib.load().qi_dit_step_cfg(ctypes.byref(model.dims), ctypes.byref(model.w), N, _ptr(img_tokens),
                                     float(t), _ptr(img_cos2), _ptr(img_sin2), ctypes.byref(cache_pos.c),
                                     ctypes.byref(cache_neg.c), _ptr(vel2), ws.ptr, ws.nbytes,
                                     stream_handle(stream))
    check(st, "qi_dit_step_cfg")


def dit_step_fbc(model: DeviceModel, L: int, N: int, img_tokens, t: float, img_cos, img_sin, cache: KVCache,
                 threshold: float, fbc: FirstBlockCache, vel, ws: Workspace, stream=None):
    """Image-only step with the first-block cache (Fast mode)."""
    st = _lib.load().qi_dit_step_fbc(ctypes.byref(model.dims), ctypes.byref(model.w), L, N, _ptr(img_tokens),
                                     float(t), _ptr(img_cos), _ptr(img_sin), ctypes.byref(cache.c),
                                     float(threshold), fbc.ptr, fbc.nbytes, _ptr(vel), ws.ptr, ws.nbytes,
                                     stream_handle(stream))
    check(st, "qi_dit_step_fbc")


def euler_update_cfg(x, vel2, guidance: float, sigma_cur: float, sigma_next: float, stream=None):
    """x += (sigma_next - sigma_cur) * (neg + g (pos - neg)), vel2 = [pos | neg]."""
    n = x.numel()
    if vel2.numel() != 2 * n:
        raise ValueError("vel2 must hold 2 * x.numel() values")
    st = _lib.load().qi_euler_update_cfg(_ptr(x), _ptr(vel2), float(guidance), float(sigma_cur),
                                         float(sigma_next), n, stream_handle(stream))
    check(st, "qi_euler_update_cfg")


def dpmpp_2m_coeffs(sigma_prev, sigma_cur: float, sigma_next: float):
    """(a, b, c1, c2, order) of one DPM++ 2M step (host, float64);
    sigma_prev None on the first step."""
    c = (ctypes.c_double * 4)()
    has = sigma_prev is not None
    r = _lib.load().qi_dpmpp_2m_coeffs(int(has), float(sigma_prev) if has else 0.0, float(sigma_cur),
                                       float(sigma_next), c)
    if r < 0:
        check(r, "qi_dpmpp_2m_coeffs")
    return c[0], c[1], c[2], c[3], int(r)


def dpmpp_2m_update(x, vel, x0_prev, sigma_prev, sigma_cur: float, sigma_next: float, stream=None):
    """In-place DPM++ 2M step; x0_prev (same size as x) carries the data
    prediction between steps; sigma_prev None on the first step."""
    n = x.numel()
    if vel.numel() != n or x0_prev.numel() != n:
        raise ValueError("x, vel and x0_prev sizes differ")
    has = sigma_prev is not None
    st = _lib.load().qi_dpmpp_2m_update(_ptr(x), _ptr(vel), _ptr(x0_prev), int(has),
                                        float(sigma_prev) if has else 0.0, float(sigma_cur), float(sigma_next),
                                        n, stream_handle(stream))
    check(st, "qi_dpmpp_2m_update")


def modulation(dims: QiDims, w_mod, b_mod, t: float, mod, stream=None):
    st = _lib.load().qi_modulation(ctypes.byref(dims), _ptr(w_mod), _ptr(b_mod), float(t), _ptr(mod),
                                   stream_handle(stream))
    check(st, "qi_modulation")


def block_causal_attention(heads: int, L: int, N: int, mode: int, q_t, k_t, vt_t, q_i, k_i, vt_i, o,
                           stream=None):
    st = _lib.load().qi_block_causal_attention(heads, L, N, mode, _ptr(q_t), _ptr(k_t), _ptr(vt_t),
                                               _ptr(q_i), _ptr(k_i), _ptr(vt_i), _ptr(o),
                                               stream_handle(stream))
    check(st, "qi_block_causal_attention")


def linear_bf16(A, W, bias, C, stream=None):
    M, K = A.shape
    N = W.shape[0]
    st = _lib.load().qi_linear_bf16(M, N, K, _ptr(A), _ptr(W), _ptr(bias), _ptr(C), stream_handle(stream))
    check(st, "qi_linear_bf16")


# ------------------------------------------------------------------ kernel timing

KERNEL_KINDS = ["modulation", "txt_norm", "gemm_txt", "img_embed", "norm_mod", "gemm_qkv", "attention",
                "gemm_o", "gemm_gate_up", "gemm_down", "head", "euler", "enc_gemm", "enc_attention", "enc_misc", "splitk_reduce"]


def timing_begin(max_launches: int = 65536):
    check(_lib.load().qi_timing_begin(int(max_launches)), "qi_timing_begin")


def timing_end() -> dict:
    """{kind: (total_ms, launches)} for the launches since timing_begin()."""
    n = _lib.QI_KERNEL_KINDS
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    dropped = ctypes.c_int64(0)
    check(_lib.load().qi_timing_end(ms, cnt, ctypes.byref(dropped)), "qi_timing_end")
    if dropped.value:
        raise RuntimeError(f"kernel timing dropped {dropped.value} launches; raise max_launches")
    lib = _lib.load()
    return {lib.qi_kernel_kind_name(k).decode(): (ms[k], int(cnt[k])) for k in range(n)}
