"""Algorithmic work of the DiT step: FLOPs of the contractions and HBM bytes
of the bandwidth-bound kernels, per launch, used to turn measured kernel
durations into roofline fractions.

FLOPs count 2 per multiply-add of the plain definition (no masked work): a
GEMM is 2 M N K; attention is 4 d per (query, key) pair that the block-causal
mask allows, pairs = N (L + N) + L (L + 1) / 2 on a joint pass and N (L + N)
on an image-only pass.  Bytes are the minimum each kernel must move: its
inputs read once and its outputs written once.  The model reproduces the
MLX page's "598 tokens through 32 blocks, about 8.5 TFLOP" ("Where the time
goes")."""
from __future__ import annotations

from dataclasses import dataclass

# MI355X published peaks (dense; no sparsity)
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


@dataclass(frozen=True)
class Shape:
    hidden: int
    ffn: int
    L: int
    N: int
    n_blocks: int
    txt_dim: int
    joint: bool

    @property
    def T(self) -> int:
        return self.L + self.N if self.joint else self.N

    @property
    def heads(self) -> int:
        return self.hidden // 128


def attention_pairs(L: int, N: int, joint: bool) -> int:
    p = N * (L + N)
    if joint:
        p += L * (L + 1) // 2
    return p


def kernel_work(s: Shape) -> dict:
    """Per-launch algorithmic work of each kernel kind: {kind: (flops, bytes)}."""
    H, F, T, N, L, D = s.hidden, s.ffn, s.T, s.N, s.L, s.txt_dim
    w = {
        "gemm_qkv": (2 * T * 3 * H * H, 2 * (T * H + 3 * H * H + 3 * T * H)),
        "attention": (4 * H * attention_pairs(L, N, s.joint), 2 * (3 * T * H + 2 * L * H * (0 if s.joint else 1) + T * H)),
        "gemm_o": (2 * T * H * H, 2 * (T * H + H * H) + 8 * T * H),
        "gemm_gate_up": (2 * T * 2 * F * H, 2 * (T * H + 2 * F * H + T * F)),
        "gemm_down": (2 * T * H * F, 2 * (T * F + H * F) + 8 * T * H),
        "norm_mod": (0, 6 * T * H),
        "modulation": (2 * 2 * 4 * H * H, 2 * 4 * H * H + 2 * 4 * H * 4),
        "img_embed": (2 * N * 64 * H, 4 * N * 64 + 2 * H * 64 + 4 * N * H),
        "head": (2 * N * H * 64, 4 * N * H + 2 * 64 * H + 4 * N * 64),
        "euler": (0, 12 * N * 64),
    }
    if s.joint:
        w["txt_norm"] = (0, 4 * L * D + 2 * L * D)
        w["gemm_txt"] = (2 * L * D * H, 2 * (L * D + H * D) + 4 * L * H)
    return w


def block_flops(s: Shape) -> int:
    """FLOPs of one block: 2 x 13 H^2 per row for F = 3H (QKV 3H^2, O H^2,
    gate/up 2FH, down FH) plus attention."""
    H, F = s.hidden, s.ffn
    return 2 * s.T * (4 * H * H + 3 * F * H) + 4 * H * attention_pairs(s.L, s.N, s.joint)


def step_flops(s: Shape, include_shared: bool = False) -> int:
    f = s.n_blocks * block_flops(s)
    if include_shared:
        kw = kernel_work(s)
        f += sum(kw[k][0] for k in ("modulation", "img_embed", "head", "gemm_txt") if k in kw)
    return f


def launches_per_step(s: Shape) -> dict:
    """Launches of each kernel kind in one step (two norms per block)."""
    n = {k: s.n_blocks for k in ("gemm_qkv", "attention", "gemm_o", "gemm_gate_up", "gemm_down")}
    n.update(norm_mod=2 * s.n_blocks, modulation=1, img_embed=1, head=1)
    if s.joint:
        n.update(txt_norm=1, gemm_txt=1)
    return n


def step_bytes(s: Shape) -> int:
    """Algorithmic HBM bytes of one step: every kernel's minimum traffic
    (kernel_work) times its launches per step, the Euler update excluded."""
    kw = kernel_work(s)
    return sum(kw[k][1] * n for k, n in launches_per_step(s).items())


def encoder_flops(hidden: int, heads: int, kv_heads: int, ffn: int, n_layers: int, L: int,
                  head_dim: int = 128) -> dict:
    """Algorithmic FLOPs of one causal forward of the text encoder over L
    tokens (no masked work, no padding): the projections 2 L (H (heads +
    2 kv_heads) d + heads d H + 3 F H) per layer and attention 4 d heads per
    allowed (query, key) pair, L (L + 1) / 2 of them."""
    H, F, d = hidden, ffn, head_dim
    gemm = 2 * L * (H * (heads + 2 * kv_heads) * d + heads * d * H + 3 * F * H) * n_layers
    attn = 4 * d * heads * (L * (L + 1) // 2) * n_layers
    return {"gemm": gemm, "attention": attn, "total": gemm + attn}
