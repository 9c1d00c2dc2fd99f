"""Plain CPU oracle of the text encoder (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library; both sides take their inputs from the
seeded generators in `qi_synth`.

Pages cited (by title and section):
  [PORT]  "Qwen-Image-2.1 port" knowledge page of the coreai-model-zoo: the
          pieces table (Text encoder row) and the fp32-compute paragraph
          ("<|im_start|> tokens need fp32 compute").
  [HOST]  "Host contract -- RGBA-Image-2.1 (Core AI port of Qwen-Image-2.1)",
          sections 1 (the encoder graph) and 3 (Encode).

What the pages fix: the Qwen3-VL-8B text stack -- 36 layers, hidden 4096,
GQA 32:8, head dim 128, MLP 12288, q_norm + k_norm, RoPE theta 5e6 which for
text alone is plain 1-D RoPE; input_ids [Lfull] -> hidden [Lfull, 4096], the
residual stream after the last layer with no final norm; embed_tokens inside;
bf16 weights with fp32 compute (w16a32); attention causal.

Readings of points the pages leave open:
  E1  the layer is the Qwen3 decoder layer: x += o_proj(attn(RMSNorm(x;
      input_layernorm))); x += down(SiLU(gate(h)) * up(h)) with h =
      RMSNorm(x; post_attention_layernorm); no biases; RMSNorm eps 1e-6.
  E2  q_norm / k_norm: RMSNorm over each head's 128 features with a learned
      128-vector, applied to q and k after the projection and before RoPE.
  E3  RoPE pairs feature i with i + 64 in each head (rotate-half):
      (a, b) -> (a c - b s, b c + a s) with c, s of angle p * theta^(-2i/128),
      i < 64, p the token's position 0..Lfull-1.  Table steps each rounded
      to fp32 (the exponent 2i/128, the power, its reciprocal, the product
      with p), pow and cos/sin correctly rounded -- the DiT tables' rule.
  E4  GQA: query head h reads key/value head h // (heads / kv_heads);
      softmax scale 1/sqrt(128); query i sees keys 0..i.
Pinned in tests/test_oracle_encoder.py against an independent implementation
of the same architecture (the Qwen3-VL text model of the transformers
library) and against closed forms.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
RMS_EPS = 1e-6


def rope_table(L: int, d: int = 128, theta: float = 5.0e6):
    """Reading E3: cos, sin [L, d/2] fp32 for positions 0..L-1."""
    half = d // 2
    expo = np.array([F32(2 * i) / F32(d) for i in range(half)], dtype=F32)        # fp32 quotient
    power = np.array([F32(math.pow(theta, float(e))) for e in expo], dtype=F32)     # pow rounded once
    inv = (F32(1.0) / power).astype(F32)
    pos = np.arange(L, dtype=F32)
    ang = (pos[:, None] * inv[None, :]).astype(F32)
    cos = np.vectorize(lambda a: F32(math.cos(float(a))), otypes=[F32])(ang)
    sin = np.vectorize(lambda a: F32(math.sin(float(a))), otypes=[F32])(ang)
    return cos.astype(F32), sin.astype(F32)


def rms_norm(v: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """v * rsqrt(mean(v^2) + eps) * w over the last axis (reading E1)."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * w


def rope_rotate_half(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Reading E3 on x [..., L, d] with cos/sin [L, d/2]."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def gqa_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Reading E4: q [heads, L, d], k/v [kv_heads, L, d] -> [heads, L, d]."""
    heads, L, d = q.shape
    group = heads // k.shape[0]
    kk = np.repeat(k, group, axis=0)
    vv = np.repeat(v, group, axis=0)
    s = q @ np.swapaxes(kk, -1, -2) / math.sqrt(d)
    s = np.where(np.triu(np.ones((L, L), dtype=bool), k=1), -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p / p.sum(axis=-1, keepdims=True)) @ vv


def encoder_layer(x: np.ndarray, lw: dict, cos: np.ndarray, sin: np.ndarray, heads: int, kv_heads: int):
    """One layer (readings E1-E4) on x [L, H]."""
    L, H = x.shape
    dt = x.dtype
    d = lw["q_norm"].shape[0]
    h = rms_norm(x, lw["in_norm"].astype(dt))
    q = (h @ lw["w_q"].astype(dt).T).reshape(L, heads, d).transpose(1, 0, 2)
    k = (h @ lw["w_k"].astype(dt).T).reshape(L, kv_heads, d).transpose(1, 0, 2)
    v = (h @ lw["w_v"].astype(dt).T).reshape(L, kv_heads, d).transpose(1, 0, 2)
    q = rope_rotate_half(rms_norm(q, lw["q_norm"].astype(dt)), cos, sin)
    k = rope_rotate_half(rms_norm(k, lw["k_norm"].astype(dt)), cos, sin)
    o = gqa_causal_attention(q, k, v).transpose(1, 0, 2).reshape(L, heads * d)
    x = x + o @ lw["w_o"].astype(dt).T
    h = rms_norm(x, lw["post_norm"].astype(dt))
    g = h @ lw["w_gate"].astype(dt).T
    u = h @ lw["w_up"].astype(dt).T
    return x + (g / (1.0 + np.exp(-g)) * u) @ lw["w_down"].astype(dt).T


def text_encoder(embed: np.ndarray, layers, ids: np.ndarray, cos: np.ndarray, sin: np.ndarray, heads: int,
                 kv_heads: int, dtype=np.float64) -> np.ndarray:
    """input_ids [L] -> hidden [L, H]: embed_tokens, the layers, no final norm
    ([HOST] s.1).  layers: an iterable of per-layer weight dicts (fp32 values
    of the bf16 weights)."""
    x = embed[np.asarray(ids, dtype=np.int64)].astype(dtype)
    for lw in layers:
        x = encoder_layer(x, lw, cos.astype(dtype), sin.astype(dtype), heads, kv_heads)
    return x


def min_token_corr(a: np.ndarray, ref: np.ndarray) -> float:
    """Minimum over tokens of the Pearson correlation of each token's hidden
    vector (the per-token gate of [PORT]'s fp32-compute paragraph)."""
    a = a.astype(np.float64) - a.mean(axis=1, keepdims=True)
    r = ref.astype(np.float64) - ref.mean(axis=1, keepdims=True)
    return float(((a * r).sum(axis=1) / np.sqrt((a * a).sum(axis=1) * (r * r).sum(axis=1))).min())
