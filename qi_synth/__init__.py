"""Seeded synthetic inputs for the single-stream DiT denoising step.

This module only draws numbers: random-init weights, noise latents, stand-in
prompt embeddings, and the workload shapes. It holds none of the method's
arithmetic, and both the CPU oracle and the HIP path take their inputs from it.

Shapes follow the graph contract of the DiT (Host contract -- RGBA-Image-2.1,
section 1 "The graphs"): img_tokens [1,N,64], txt_feats [1,L,4096], a scalar
timestep, fp32 at the boundary.  There are no real weights: every Linear weight
and bias is N(0, 0.02), every RMSNorm weight 1 + N(0, 0.02), and the
zero-centred text-norm weight N(0, 0.02).  Each tensor has its own numpy PCG64
stream seeded by SeedSequence([master, block, tensor_id]), so one block can be
regenerated alone and a one-block workload shares block 0 with the 32-block
ones.  For bf16 workloads the values are rounded once, round-to-nearest-even,
and handed out as bf16 bit patterns (uint16).

The initial latent is drawn the way the host contract draws it (section 5
"Noise and pack"): torch.randn((1,1,64,h,w)) from a CPU generator with the
given seed, packed token-major as x[y*w + x, c] = z[c, y, x].  The prompt
embeddings are N(0,1) stand-ins of the pages' prompt lengths; the pages hold
no public benchmark or dataset for the DiT.
"""
from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass, field, replace

import numpy as np

MASTER_SEED = 0
SHARED_BLOCK_ID = 100000          # stream id for the tensors outside the blocks
NOISE_SEED = 1234                 # the seed of the Core AI port's oracle run
TXT_SEED = 1235
NEG_TXT_SEED = 1236               # the negative prompt of a true-CFG render

# tensor ids inside a block
_BLOCK_TENSORS = ("w_qkv", "w_o", "w_gu", "w_down", "norm1", "norm2")
# tensor ids of the shared pieces
_SHARED_TENSORS = ("w_mod", "b_mod", "w_img", "b_img", "txt_norm", "w_txt",
                   "b_txt", "norm_out", "w_out", "b_out")

LIN_STD = 0.02


@dataclass(frozen=True)
class Workload:
    """One DiT workload: model width/depth and the [text L | image N] shape."""
    name: str
    hidden: int
    ffn: int
    L: int
    h: int
    w: int
    n_blocks: int
    bf16_weights: bool
    txt_dim: int
    head_dim: int = 128
    timestep: float = 0.7
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def heads(self) -> int:
        return self.hidden // self.head_dim

    @property
    def N(self) -> int:
        return self.h * self.w

    @property
    def T_joint(self) -> int:
        return self.L + self.N


# The five workloads: a reduced CPU-sized block, one full-width block, and the
# full 32-block model at 384^2 (L=494), 1024^2 (L=407) and 2048^2 (L=512).
WORKLOADS = {
    1: Workload("reduced-1blk-h512-L8-N64", 512, 1536, 8, 8, 8, 1, False, 512),
    2: Workload("block-h4096-L22-N256", 4096, 12288, 22, 16, 16, 1, True, 4096),
    3: Workload("dit32-384px-L494-N576", 4096, 12288, 494, 24, 24, 32, True, 4096),
    4: Workload("dit32-1024px-L407-N4096", 4096, 12288, 407, 64, 64, 32, True, 4096),
    5: Workload("dit32-2048px-L512-N16384", 4096, 12288, 512, 128, 128, 32, True, 4096),
}


def workload(k: int, **over) -> Workload:
    wl = WORKLOADS[k]
    return replace(wl, **over) if over else wl


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even, returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- streams

def _rng(block: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([MASTER_SEED, block, tensor_id])))


def _normal(block: int, tensor_id: int, shape, std: float, offset: float = 0.0) -> np.ndarray:
    g = _rng(block, tensor_id)
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    a *= np.float32(std)
    if offset:
        a += np.float32(offset)
    return a


def _block_shapes(wl: Workload):
    H, F = wl.hidden, wl.ffn
    return {
        "w_qkv": ((3 * H, H), LIN_STD, 0.0),
        "w_o": ((H, H), LIN_STD, 0.0),
        "w_gu": ((2 * F, H), LIN_STD, 0.0),
        "w_down": ((H, F), LIN_STD, 0.0),
        "norm1": ((H,), LIN_STD, 1.0),
        "norm2": ((H,), LIN_STD, 1.0),
    }


def _shared_shapes(wl: Workload):
    H, D = wl.hidden, wl.txt_dim
    return {
        "w_mod": ((4 * H, H), LIN_STD, 0.0),
        "b_mod": ((4 * H,), LIN_STD, 0.0),
        "w_img": ((H, 64), LIN_STD, 0.0),
        "b_img": ((H,), LIN_STD, 0.0),
        "txt_norm": ((D,), LIN_STD, 0.0),
        "w_txt": ((H, D), LIN_STD, 0.0),
        "b_txt": ((H,), LIN_STD, 0.0),
        "norm_out": ((H,), LIN_STD, 1.0),
        "w_out": ((64, H), LIN_STD, 0.0),
        "b_out": ((64,), LIN_STD, 0.0),
    }


# Linear weights (2-D) go to the device as bf16; vectors (biases, norm
# weights) stay fp32 on both sides.
def _draw(block: int, names, shapes, as_bf16: bool, threads: int):
    def one(item):
        idx, name = item
        shape, std, off = shapes[name]
        a = _normal(block, idx, shape, std, off)
        if len(shape) == 2 and as_bf16:
            return name, f32_to_bf16_bits(a)
        return name, a

    items = list(enumerate(names))
    if threads > 1:
        with _cf.ThreadPoolExecutor(threads) as ex:
            return dict(ex.map(one, items))
    return dict(one(i) for i in items)


def block_weights(wl: Workload, b: int, as_bf16: bool | None = None, threads: int = 4) -> dict:
    """Weights of block b.  2-D weights are uint16 bf16 bits when as_bf16
    (default: the workload's weight type), else float32."""
    if as_bf16 is None:
        as_bf16 = wl.bf16_weights
    return _draw(b, _BLOCK_TENSORS, _block_shapes(wl), as_bf16, threads)


def shared_weights(wl: Workload, as_bf16: bool | None = None, threads: int = 4) -> dict:
    if as_bf16 is None:
        as_bf16 = wl.bf16_weights
    return _draw(SHARED_BLOCK_ID, _SHARED_TENSORS, _shared_shapes(wl), as_bf16, threads)


def weights_as_f32(wd: dict) -> dict:
    """bf16 bit patterns -> exact float32 values (other arrays unchanged)."""
    return {k: (bf16_bits_to_f32(v) if v.dtype == np.uint16 else v) for k, v in wd.items()}


# ---------------------------------------------------------------- inputs

def noise_latent(h: int, w: int, seed: int = NOISE_SEED) -> np.ndarray:
    """Packed N(0,1) latent [h*w, 64] float32: randn((1,1,64,h,w)) from a CPU
    generator, then x[y*w+x, c] = z[c, y, x]."""
    import torch
    g = torch.Generator("cpu").manual_seed(int(seed))
    z = torch.randn((1, 1, 64, h, w), generator=g, dtype=torch.float32)
    return z.view(64, h * w).transpose(0, 1).contiguous().numpy()


def img_tokens(wl: Workload, seed: int = NOISE_SEED) -> np.ndarray:
    return noise_latent(wl.h, wl.w, seed)


def txt_feats(wl: Workload, seed: int = TXT_SEED, L: int | None = None) -> np.ndarray:
    """N(0,1) stand-in prompt embeddings [L, txt_dim] float32."""
    L = wl.L if L is None else L
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    return g.standard_normal((L, wl.txt_dim), dtype=np.float32)


def normal_array(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Generic N(0, scale^2) float32 array for kernel-level tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def neg_prompt_len(wl: Workload) -> int:
    """Length of the stand-in negative prompt of a true-CFG render: half the
    positive prompt (at least 1), so the two K/V slots differ in L."""
    return max(1, wl.L // 2)


def neg_txt_feats(wl: Workload) -> np.ndarray:
    """N(0,1) stand-in negative-prompt embeddings [neg_prompt_len, txt_dim]."""
    return txt_feats(wl, seed=NEG_TXT_SEED, L=neg_prompt_len(wl))


# ---------------------------------------------------------------- text encoder

@dataclass(frozen=True)
class EncWorkload:
    """A Qwen3-VL-8B-style text stack: width, GQA heads, depth, vocabulary and
    the full prompt length Lfull (system prefix included)."""
    name: str
    hidden: int
    heads: int
    kv_heads: int
    ffn: int
    n_layers: int
    vocab: int
    L_full: int
    head_dim: int = 128
    rope_theta: float = 5.0e6


# 1: CPU-oracle size; 2: full width, 2 layers, the pages' oracle length 32;
# 3: the full 36-layer stack at the 1024^2 prompt (407 DiT tokens + 14).
ENC_WORKLOADS = {
    1: EncWorkload("enc-reduced-h512-2L-L24", 512, 4, 1, 1536, 2, 1024, 24),
    2: EncWorkload("enc-h4096-2L-L32", 4096, 32, 8, 12288, 2, 151936, 32),
    3: EncWorkload("enc36-L421", 4096, 32, 8, 12288, 36, 151936, 421),
}

ENC_LAYER_BASE = 200000           # stream id of encoder layer i: ENC_LAYER_BASE + i
ENC_EMBED_ID = 300000
ENC_IDS_SEED = 1237
# the system part of the text-to-image template, as token ids (host contract, s.2)
SYSTEM_PREFIX_IDS = (151644, 8948, 198, 1092, 30782, 408, 323, 23643, 279, 3897, 9934, 13, 151645, 198)

_ENC_TENSORS = ("w_q", "w_k", "w_v", "q_norm", "k_norm", "w_o", "w_gate", "w_up", "w_down", "in_norm",
                "post_norm")


def enc_workload(k: int, **over) -> EncWorkload:
    ew = ENC_WORKLOADS[k]
    return replace(ew, **over) if over else ew


def _enc_shapes(ew: EncWorkload):
    H, F, d = ew.hidden, ew.ffn, ew.head_dim
    return {
        "w_q": ((ew.heads * d, H), LIN_STD, 0.0),
        "w_k": ((ew.kv_heads * d, H), LIN_STD, 0.0),
        "w_v": ((ew.kv_heads * d, H), LIN_STD, 0.0),
        "q_norm": ((d,), LIN_STD, 1.0),
        "k_norm": ((d,), LIN_STD, 1.0),
        "w_o": ((H, ew.heads * d), LIN_STD, 0.0),
        "w_gate": ((F, H), LIN_STD, 0.0),
        "w_up": ((F, H), LIN_STD, 0.0),
        "w_down": ((H, F), LIN_STD, 0.0),
        "in_norm": ((H,), LIN_STD, 1.0),
        "post_norm": ((H,), LIN_STD, 1.0),
    }


def enc_layer_weights(ew: EncWorkload, layer: int, as_bf16: bool = True, threads: int = 4) -> dict:
    """Weights of encoder layer `layer` (2-D ones as bf16 bits when as_bf16)."""
    return _draw(ENC_LAYER_BASE + layer, _ENC_TENSORS, _enc_shapes(ew), as_bf16, threads)


def enc_embed(ew: EncWorkload, as_bf16: bool = True) -> np.ndarray:
    """Token embedding table [vocab, hidden], N(0, 0.02)."""
    a = _normal(ENC_EMBED_ID, 0, (ew.vocab, ew.hidden), LIN_STD)
    return f32_to_bf16_bits(a) if as_bf16 else a


def enc_input_ids(ew: EncWorkload, seed: int = ENC_IDS_SEED, L: int | None = None) -> np.ndarray:
    """int32 ids [L]: the printed system prefix when the vocabulary holds it,
    then seeded uniform ids."""
    L = ew.L_full if L is None else L
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed])))
    ids = g.integers(0, ew.vocab, size=L, dtype=np.int64)
    if ew.vocab > max(SYSTEM_PREFIX_IDS) and L >= len(SYSTEM_PREFIX_IDS):
        ids[:len(SYSTEM_PREFIX_IDS)] = SYSTEM_PREFIX_IDS
    return ids.astype(np.int32)
