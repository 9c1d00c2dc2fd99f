"""Plain CPU oracle of the single-stream DiT denoising step (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark do.  It shares no code with the HIP library; both sides take
their inputs from the seeded generators in `qi_synth`.

Pages cited (by title and section):
  [PORT]  "Qwen-Image-2.1 port" knowledge page of the coreai-model-zoo
          (the pieces table, DiT row; the Oracle and gate paragraphs).
  [HOST]  "Host contract -- RGBA-Image-2.1 (Core AI port of Qwen-Image-2.1)",
          sections 1-6.
  [MLX]   "Qwen-Image-2.1 on MLX, faster and exact", sections "Text K/V reuse
          (exact, on by default)", "Where the time goes" and "Optional modes
          (approximate or slower)", including its Fast mode.

Floating point: the DiT forward runs in float64 (the `dtype` argument can
lower it).  The RoPE tables, the sampler arrays and the Euler update are fp32
because the host contract fixes them as fp32 ([HOST] sections 4 and 6).

Readings of points the pages leave open (each is stated where it is used):
  S1  time embedding: width-H sinusoid [cos | sin] of 1000*t, frequencies
      10000^(-j/(H/2)); no time MLP.
  S2  the 4H modulation row splits into (scale1, gate1, scale2, gate2); norm
      output is multiplied by (1 + scale), residual branch by the raw gate.
  S3  RMSNorm eps 1e-6 with a learned weight.
  S4  ZeroCenterRMSNorm = v * rsqrt(mean(v^2) + eps) * (1 + w).
  S5  text projection = Linear(D_txt -> H) with bias.
  S6  block Linears carry no bias; embed, text projection, modulation and
      proj_out do.
  S7  SDPA scale 1/sqrt(128); a text row sees text keys 0..i inclusive.
  S8  "interleaved" RoPE: adjacent pairs (2k, 2k+1) of each head form complex
      number k; applied to q and k, not v; no q/k norm.
  S9  final layer = RMSNorm then Linear(H -> 64) with bias, image rows only.
  S10 SwiGLU: rows [0,F) of the gate/up weight are the gate (SiLU), [F,2F)
      the up projection.
  S11 precision: the host contract fixes the DiT as "bf16 weights and
      compute, fp32 boundary" without listing rounding points.  exact mode
      (default) computes the definition in float64; bf16 mode (bf16=True)
      rounds every matmul operand once to bf16 (round to nearest even) --
      the block's normed inputs, q, k, v after RoPE, the attention
      probabilities (relative to the row max), the attention output, the
      SwiGLU output and the normed text features -- with fp32-or-better
      accumulation, residual stream, norm statistics and softmax sums.
  S12 RoPE tables: each step of the printed formula rounded to fp32, pow and
      cos/sin correctly rounded (evaluated in float64, rounded once).
  S13 metrics: rel L2 over all of vel; per-token Pearson correlation over the
      64 channels, minimum over tokens.
  S14 Euler: the sigma difference in fp32, then a fp32 multiply and a fp32
      add, no fused multiply-add.
  S15 sampler constants base_shift 0.5 at 256 tokens, max_shift 0.9 at 8192
      tokens, mu linear in N with no clamp, 1000 train timesteps; each array
      operation in fp32 as the host contract states, mu and e^mu in float64.
  S16 image frame position: the first position axis of every image token is
      L, the text length, as the host contract prints it.
  S20 true CFG: noise = neg + g * (pos - neg) exactly as [MLX] "Optional
      modes" writes it (no rescaling of the combined prediction), evaluated
      in fp32 as written -- difference, product, sum, each rounded once -- and
      fed to the S14 Euler update; each branch is an ordinary step on its own
      prompt (its own text K/V and its own image RoPE rows, which depend on
      its L).
  S21 first-block cache (Fast mode): block 0 always runs; its residual
      r0 = x1 - x0 (after the embed, after block 0) is compared with the r0
      cached at the last step that ran every block, change = sum|r0 - r0c| /
      sum|r0c| over all image rows and features; below the threshold blocks
      1.. are skipped and x = x1 + remc, the residual x_out - x1 that blocks
      1.. produced at that last full step; otherwise they run and r0, remc
      are cached.  (The page says only that blocks 1.. are skipped while block
      0's residual changes less than the threshold; comparing against the last
      full step rather than the previous step keeps slow drift from adding up
      unchecked, and reusing the last full step's residual is the plainest
      value for the skipped work.)
  S22 DPM++ 2M sampler: the page only names it.  Read as DPM-Solver++(2M)
      (Lu et al., "DPM-Solver++: Fast Solver for Guided Sampling of
      Diffusion Probabilistic Models", 2022, the multistep second-order
      data-prediction solver) written for the flow x = (1 - sigma) x0 +
      sigma eps: alpha = 1 - sigma, lambda = log(alpha / sigma), data
      prediction x0 = x - sigma * v.  Step sigma_s -> sigma_t with
      h = lambda_t - lambda_s:
        x_t = (sigma_t / sigma_s) x_s - alpha_t (e^-h - 1) D,
        D = x0_s (first order) or (1 + 1/(2r)) x0_s - 1/(2r) x0_prev with
        r = h_prev / h (second order);
      first order at the first step and at the final step (sigma_t = 0,
      where h is infinite), as the reference implementations of the method
      do; the same FlowMatch sigmas as Euler.  Coefficients in float64; the
      update in fp32 in the order p = sigma_s v, x0 = x - p, D = c1 x0 -
      c2 x0_prev, x_t = a x - b D (each operation rounded once).
Parity pins live in tests/test_oracle_*.py.  The whole-step vel has no
printed value on the pages: beyond the invariants and component pins it is
"parity unpinned" externally.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128
ROPE_AXES = (16, 56, 56)          # head-dim split per axis [PORT] DiT row; [HOST] s.4
ROPE_POS_MIN, ROPE_POS_MAX = -1024, 8191   # table rows [HOST] s.4
RMS_EPS = 1e-6                    # S3

F32 = np.float32


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), keeping a's dtype:
    the 16 high bits of the float32 representation after rounding."""
    u = np.array(a, dtype=np.float32, copy=True, order="C").view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))  # wraps like the 32-bit word
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(a.dtype, copy=False)


# ------------------------------------------------------------------ RoPE

def rope_axis_table(d: int):
    """fp32 cos/sin table of one axis ([HOST] s.4): row p + 1024 for each
    position p in -1024..8191; column k is the unit complex number at angle
    p * w_k with inverse frequency w_k = 1 / 10000^(2k/d).  Reading S12 for
    the rounding."""
    pos = np.arange(ROPE_POS_MIN, ROPE_POS_MAX + 1, dtype=np.int64)
    expo = np.arange(0, d, 2, dtype=np.int64).astype(F32) / F32(d)          # fp32 quotient
    powv = np.power(np.float64(10000.0), expo.astype(np.float64)).astype(F32)  # pow, rounded once
    freq = F32(1.0) / powv                                                  # fp32 reciprocal
    ang = pos.astype(F32)[:, None] * freq[None, :]                          # fp32 product
    a64 = ang.astype(np.float64)
    return np.cos(a64).astype(F32), np.sin(a64).astype(F32)


def token_positions(L: int, h: int, w: int):
    """3-axis positions ([HOST] s.4): text token i -> (i, i, i); image token
    (y, x) at index y*w + x -> (L, y - (h - h//2), x - (w - w//2))."""
    txt = np.repeat(np.arange(L, dtype=np.int64)[:, None], 3, axis=1)
    yy, xx = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    img = np.stack([np.full(h * w, L, dtype=np.int64),
                    (yy.reshape(-1) - (h - h // 2)),
                    (xx.reshape(-1) - (w - w // 2))], axis=1)
    return txt, img


def rope_rows(L: int, h: int, w: int):
    """Per-token 64-wide cos/sin rows: the three axis rows concatenated in
    axis order, 8 + 28 + 28 values ([HOST] s.4).  Returns (txt_cos, txt_sin,
    img_cos, img_sin) as fp32 [L,64], [L,64], [N,64], [N,64]."""
    tabs = [rope_axis_table(d) for d in ROPE_AXES]
    txt, img = token_positions(L, h, w)

    def gather(pos):
        cs = [tabs[a][0][pos[:, a] - ROPE_POS_MIN] for a in range(3)]
        sn = [tabs[a][1][pos[:, a] - ROPE_POS_MIN] for a in range(3)]
        return np.concatenate(cs, axis=1), np.concatenate(sn, axis=1)

    tc, ts = gather(txt)
    ic, is_ = gather(img)
    return tc, ts, ic, is_


def rope_apply(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (reading S8): for rows r, heads, k = 0..63,
    (a, b) = (x[r,h,2k], x[r,h,2k+1]) -> (a c - b s, a s + b c) with
    (c, s) = (cos[r,k], sin[r,k]).  x is [T, heads, 128]."""
    out = np.empty_like(x)
    c = cos.astype(x.dtype)[:, None, :]
    s = sin.astype(x.dtype)[:, None, :]
    a = x[:, :, 0::2]
    b = x[:, :, 1::2]
    out[:, :, 0::2] = a * c - b * s
    out[:, :, 1::2] = a * s + b * c
    return out


# ------------------------------------------------------------------ time / modulation

def timestep_embedding(tau: float, H: int, dtype=np.float64) -> np.ndarray:
    """Reading S1: e[j] = cos(1000 tau f_j), e[H/2 + j] = sin(1000 tau f_j),
    f_j = 10000^(-j/(H/2)), j < H/2."""
    half = H // 2
    j = np.arange(half, dtype=np.float64)
    f = np.power(10000.0, -j / half)
    arg = 1000.0 * float(tau) * f
    return np.concatenate([np.cos(arg), np.sin(arg)]).astype(dtype)


def modulation_rows(w_mod, b_mod, t: float, H: int, dtype=np.float64):
    """The one modulation Linear shared by all blocks, evaluated for t = 0
    (text rows) and for the sampled t (image rows) ([PORT] DiT row; [MLX]
    "Text K/V reuse").  Returns (m_txt, m_img), each [4H]."""
    W = w_mod.astype(dtype)
    b = b_mod.astype(dtype)
    m_txt = W @ timestep_embedding(0.0, H, dtype) + b
    m_img = W @ timestep_embedding(t, H, dtype) + b
    return m_txt, m_img


def split_mod(m: np.ndarray, H: int):
    """Reading S2: chunk order (scale1, gate1, scale2, gate2)."""
    return m[0:H], m[H:2 * H], m[2 * H:3 * H], m[3 * H:4 * H]


# ------------------------------------------------------------------ norms / MLP

def rms_norm(v: np.ndarray, gamma: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """v * rsqrt(mean(v^2) + eps) * gamma over the last axis (S3)."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * gamma.astype(v.dtype)


def zero_center_rms_norm(v: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Reading S4 of the text projection's ZeroCenterRMSNorm ([PORT] DiT row)."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * (1.0 + w.astype(v.dtype))


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


# ------------------------------------------------------------------ attention

def sdpa(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, bf16: bool = False) -> np.ndarray:
    """Scaled dot-product attention for one segment, [heads, Tq, d] x
    [heads, Tk, d] -> [heads, Tq, d], scale 1/sqrt(d) (S7).  causal: query i
    sees keys 0..i (requires Tq == Tk).  bf16 (reading S11): the
    probabilities relative to the row max are rounded to bf16 before they
    multiply v; the normalising sum uses the unrounded values."""
    d = q.shape[-1]
    mask = np.triu(np.ones((q.shape[1], k.shape[1]), dtype=bool), k=1) if causal else None
    out = np.empty(q.shape[:2] + (v.shape[-1],), dtype=np.result_type(q, k, v))
    # one head at a time (the heads are independent; this keeps one head's
    # [Tq, Tk] scores in memory, 2.3 GB in float64 at 16896 tokens)
    for hd in range(q.shape[0]):
        s = np.matmul(q[hd], k[hd].T) / math.sqrt(d)
        if causal:
            s = np.where(mask, -np.inf, s)
        s = s - np.max(s, axis=-1, keepdims=True)
        p = np.exp(s)
        l = np.sum(p, axis=-1, keepdims=True)
        if bf16:
            p = round_bf16(p)
        out[hd] = np.matmul(p, v[hd]) / l
    return out


def block_causal_attention(q_txt, k_txt, v_txt, q_img, k_img, v_img, bf16: bool = False):
    """The two-SDPA decomposition of block-causal attention ([PORT] DiT row:
    text->text causal, image->all; [MLX] "Text K/V reuse": text rows never see
    the image).  Inputs [heads, T_seg, d]; q_txt may have zero rows (an
    image-only step).  Returns (o_txt, o_img)."""
    o_txt = sdpa(q_txt, k_txt, v_txt, causal=True, bf16=bf16) if q_txt.shape[1] else q_txt.copy()
    k_all = np.concatenate([k_txt, k_img], axis=1)
    v_all = np.concatenate([v_txt, v_img], axis=1)
    o_img = sdpa(q_img, k_all, v_all, causal=False, bf16=bf16)
    return o_txt, o_img


# ------------------------------------------------------------------ block / step

def dit_block(x: np.ndarray, L_rows: int, bw: dict, m_txt, m_img, cos, sin,
              heads: int, kv_text=None, bf16: bool = False):
    """One single-stream block ([PORT] pieces table, DiT row).

    x: [T, H] residual stream, rows [text L_rows | image].  L_rows = L for a
    joint pass, 0 for an image-only pass (then kv_text = (k_txt, v_txt) from
    the cache, [heads, L, 128] each).  cos/sin: [T, 64] rows of those tokens.
    Returns (x_new, (k_txt, v_txt)) where the pair is this pass's text K/V
    (joint) or the cached pair passed in (image-only).  bf16: reading S11."""
    dt = x.dtype
    rb = round_bf16 if bf16 else (lambda a: a)
    T, H = x.shape
    mt, mi = split_mod(m_txt.astype(dt), H), split_mod(m_img.astype(dt), H)
    is_txt = (np.arange(T) < L_rows)[:, None]

    def mrow(i):
        return np.where(is_txt, mt[i][None, :], mi[i][None, :])

    s1, g1, s2, g2 = mrow(0), mrow(1), mrow(2), mrow(3)

    h = rb(rms_norm(x, bw["norm1"]) * (1.0 + s1))
    qkv = h @ bw["w_qkv"].astype(dt).T                                  # [T, 3H]
    q = qkv[:, 0:H].reshape(T, heads, HEAD_DIM)
    k = qkv[:, H:2 * H].reshape(T, heads, HEAD_DIM)
    v = rb(qkv[:, 2 * H:3 * H].reshape(T, heads, HEAD_DIM))
    q = rb(rope_apply(q, cos, sin))
    k = rb(rope_apply(k, cos, sin))
    qh, kh, vh = (np.ascontiguousarray(a.transpose(1, 0, 2)) for a in (q, k, v))

    if L_rows > 0:
        k_txt, v_txt = kh[:, :L_rows], vh[:, :L_rows]
    else:
        k_txt, v_txt = (a.astype(dt) for a in kv_text)
    o_txt, o_img = block_causal_attention(qh[:, :L_rows], k_txt, v_txt,
                                          qh[:, L_rows:], kh[:, L_rows:], vh[:, L_rows:], bf16=bf16)
    o = rb(np.concatenate([o_txt, o_img], axis=1).transpose(1, 0, 2).reshape(T, H))

    x = x + g1 * (o @ bw["w_o"].astype(dt).T)
    h2 = rb(rms_norm(x, bw["norm2"]) * (1.0 + s2))
    u = h2 @ bw["w_gu"].astype(dt).T
    F = u.shape[1] // 2
    a = rb(silu(u[:, :F]) * u[:, F:])
    x = x + g2 * (a @ bw["w_down"].astype(dt).T)
    return x, (k_txt, v_txt)


def dit_block_rows(x: np.ndarray, L_rows: int, bw: dict, m_txt, m_img, cos, sin, heads: int,
                   rows, kv_text=None):
    """dit_block evaluated for the output rows `rows` only (indices into x):
    the keys and values of every row, then attention, the output projection
    and the MLP of the selected rows, with the same definition as dit_block.
    Returns x_new[rows]."""
    dt = x.dtype
    T, H = x.shape
    rows = np.asarray(rows)
    mt, mi = split_mod(m_txt.astype(dt), H), split_mod(m_img.astype(dt), H)
    is_txt_all = (np.arange(T) < L_rows)[:, None]
    s1 = np.where(is_txt_all, mt[0][None, :], mi[0][None, :])
    h = rms_norm(x, bw["norm1"]) * (1.0 + s1)
    w_qkv = bw["w_qkv"].astype(dt)
    kv = h @ w_qkv[H:3 * H].T                                            # [T, 2H]
    k = rope_apply(kv[:, :H].reshape(T, heads, HEAD_DIM), cos, sin)
    v = kv[:, H:].reshape(T, heads, HEAD_DIM)
    q = rope_apply((h[rows] @ w_qkv[0:H].T).reshape(len(rows), heads, HEAD_DIM), cos[rows], sin[rows])
    kh, vh = (np.ascontiguousarray(a.transpose(1, 0, 2)) for a in (k, v))
    if L_rows > 0:
        k_txt, v_txt = kh[:, :L_rows], vh[:, :L_rows]
    else:
        k_txt, v_txt = (a.astype(dt) for a in kv_text)
    k_all = np.concatenate([k_txt, kh[:, L_rows:]], axis=1)
    v_all = np.concatenate([v_txt, vh[:, L_rows:]], axis=1)
    o = np.empty((len(rows), heads, HEAD_DIM), dtype=dt)
    for i, r in enumerate(rows):
        if r < L_rows:      # text row: causal over text keys 0..r
            kk, vv = k_txt[:, :r + 1], v_txt[:, :r + 1]
        else:               # image row: every text key, then every image key
            kk, vv = k_all, v_all
        o[i] = sdpa(q[i][:, None, :], kk, vv, causal=False)[:, 0, :]
    o = o.reshape(len(rows), H)
    is_txt = (rows < L_rows)[:, None]

    def mrow(j):
        return np.where(is_txt, mt[j][None, :], mi[j][None, :])

    g1, s2, g2 = mrow(1), mrow(2), mrow(3)
    xr = x[rows] + g1 * (o @ bw["w_o"].astype(dt).T)
    h2 = rms_norm(xr, bw["norm2"]) * (1.0 + s2)
    u = h2 @ bw["w_gu"].astype(dt).T
    F = u.shape[1] // 2
    a = silu(u[:, :F]) * u[:, F:]
    return xr + g2 * (a @ bw["w_down"].astype(dt).T)


def embed(sw: dict, img_tokens: np.ndarray, txt_feats, dtype=np.float64, bf16: bool = False):
    """img-in Linear(64 -> H) on the image tokens; for a joint pass also the
    text projection ZeroCenterRMSNorm -> Linear(D -> H) (readings S4, S5).
    Returns x [T, H] with rows [text | image] (text omitted if txt_feats is
    None)."""
    x_img = img_tokens.astype(dtype) @ sw["w_img"].astype(dtype).T + sw["b_img"].astype(dtype)
    if txt_feats is None:
        return x_img
    e = zero_center_rms_norm(txt_feats.astype(dtype), sw["txt_norm"])
    if bf16:
        e = round_bf16(e)
    x_txt = e @ sw["w_txt"].astype(dtype).T + sw["b_txt"].astype(dtype)
    return np.concatenate([x_txt, x_img], axis=0)


def head(sw: dict, x_img: np.ndarray) -> np.ndarray:
    """Reading S9: vel = RMSNorm(x_img; norm_out) W_out^T + b_out -> [N, 64]."""
    dt = x_img.dtype
    return rms_norm(x_img, sw["norm_out"]) @ sw["w_out"].astype(dt).T + sw["b_out"].astype(dt)


def dit_step(sw: dict, blocks, L: int, img_tokens, txt_feats, t: float,
             txt_cos, txt_sin, img_cos, img_sin, heads: int,
             kv_cache=None, capture: bool = False, dtype=np.float64,
             return_x: bool = False, bf16: bool = False):
    """One DiT forward: img_tokens [N,64], txt_feats [L,D], t -> vel [N,64]
    (the DiT graph contract, [HOST] s.1).

    blocks: a sequence (or iterable / callable b -> dict) of block weights.
    kv_cache None: joint pass over [text | image] (full recompute).
    kv_cache list of (k_txt, v_txt) per block: image rows only, text K/V read
    from the cache ([MLX] "Text K/V reuse").  capture=True returns the joint
    pass's text K/V per block as well.
    bf16: the bf16-compute reading S11 (default: exact).
    Returns vel, or (vel, cache) when capture, plus x when return_x."""
    H = sw["w_img"].shape[0]
    n_blocks = len(blocks) if hasattr(blocks, "__len__") else None
    m_txt, m_img = modulation_rows(sw["w_mod"], sw["b_mod"], t, H, dtype)
    joint = kv_cache is None
    x = embed(sw, img_tokens, txt_feats if joint else None, dtype, bf16=bf16)
    L_rows = L if joint else 0
    if joint:
        cos = np.concatenate([txt_cos, img_cos], axis=0)
        sin = np.concatenate([txt_sin, img_sin], axis=0)
    else:
        cos, sin = img_cos, img_sin
    cache = []
    it = blocks() if callable(blocks) else blocks
    for b, bw in enumerate(it):
        kv = None if joint else kv_cache[b]
        x, kv_out = dit_block(x, L_rows, bw, m_txt, m_img, cos, sin, heads, kv, bf16=bf16)
        if capture:
            cache.append(kv_out)
    if n_blocks is not None and not joint:
        assert len(kv_cache) == n_blocks
    vel = head(sw, x[L_rows:])
    out = (vel, cache) if capture else vel
    if return_x:
        return out, x
    return out


# ------------------------------------------------------------------ sampler

BASE_SHIFT, MAX_SHIFT = 0.5, 0.9            # S15
BASE_SEQ, MAX_SEQ = 256, 8192
SHIFT_TERMINAL = 0.02                       # [PORT] Sampler row; [HOST] s.6
NUM_TRAIN_TIMESTEPS = 1000


def flow_mu(n_tokens: int) -> float:
    """mu = N m + b, m = (max_shift - base_shift)/(max_seq - base_seq),
    b = base_shift - m base_seq ([HOST] s.6), constants by reading S15."""
    m = (MAX_SHIFT - BASE_SHIFT) / (MAX_SEQ - BASE_SEQ)
    b = BASE_SHIFT - m * BASE_SEQ
    return n_tokens * m + b


def flow_sigmas(steps: int, n_tokens: int):
    """FlowMatch Euler schedule ([HOST] s.6): a uniform grid from 1 down to
    1/steps; the exponential time shift s -> e^mu / (e^mu + 1/s - 1) with mu
    from flow_mu; an affine stretch of 1 - s that puts the last value at the
    terminal 0.02; timesteps = 1000 s; a final sigma 0 appended.  The host
    contract keeps these arrays in fp32 and gates them bit for bit, so each
    array operation here is one fp32 operation, and mu and e^mu are computed
    in float64 and rounded once.  Returns (sigmas fp32 [steps+1], timesteps
    fp32 [steps])."""
    s = np.linspace(1.0, 1.0 / steps, steps).astype(F32)
    em = F32(math.exp(flow_mu(n_tokens)))
    one = F32(1.0)
    s = em / (em + (one / s - one))
    s = one - (one - s) / ((one - s[-1]) / (one - F32(SHIFT_TERMINAL)))
    ts = s * F32(NUM_TRAIN_TIMESTEPS)
    return np.concatenate([s, np.zeros(1, F32)]).astype(F32), ts.astype(F32)


def timestep_input(timesteps: np.ndarray, i: int) -> np.float32:
    """t = timesteps[i] / 1000 in fp32, the DiT's timestep input ([HOST] s.6)."""
    return F32(timesteps[i]) / F32(NUM_TRAIN_TIMESTEPS)


def euler_update(x: np.ndarray, vel: np.ndarray, sigma_cur, sigma_next) -> np.ndarray:
    """x + (sigma_next - sigma_cur) * vel in fp32 ([HOST] s.6), reading S14:
    difference, product and sum each rounded to fp32 (numpy never fuses)."""
    ds = F32(sigma_next) - F32(sigma_cur)
    return (x.astype(F32) + (ds * vel.astype(F32)).astype(F32)).astype(F32)


def dpmpp_2m_coeffs(sigma_prev, sigma_cur, sigma_next):
    """Float64 coefficients (a, b, c1, c2, order) of one DPM++ 2M step
    sigma_cur -> sigma_next (reading S22): x_next = a x - b D, D = c1 x0 -
    c2 x0_prev.  sigma_prev None: no previous data prediction (first step)."""
    def lam(sg):
        sg = float(sg)
        if sg >= 1.0:
            return -math.inf
        return math.log1p(-sg) - math.log(sg)

    s_cur, s_next = float(sigma_cur), float(sigma_next)
    if s_next <= 0.0:                              # final step: x_next = x0
        return 0.0, -1.0, 1.0, 0.0, 1
    h = lam(s_next) - lam(s_cur)
    a = s_next / s_cur
    b = (1.0 - s_next) * math.expm1(-h)
    if sigma_prev is None:
        return a, b, 1.0, 0.0, 1
    r = (lam(s_cur) - lam(sigma_prev)) / h
    if math.isinf(r):                              # previous sigma was 1 (alpha 0)
        return a, b, 1.0, 0.0, 1
    c2 = 1.0 / (2.0 * r)
    return a, b, 1.0 + c2, c2, 2


def dpmpp_2m_step(x, vel, x0_prev, sigma_prev, sigma_cur, sigma_next):
    """One DPM++ 2M update in fp32 (reading S22).  Returns (x_next, x0), x0
    being the data prediction to pass as x0_prev to the next step."""
    a, b, c1, c2, order = dpmpp_2m_coeffs(sigma_prev, sigma_cur, sigma_next)
    x = x.astype(F32)
    p = (F32(sigma_cur) * vel.astype(F32)).astype(F32)
    x0 = (x - p).astype(F32)
    if order == 1:
        d = x0
    else:
        d = ((F32(c1) * x0).astype(F32) - (F32(c2) * x0_prev.astype(F32)).astype(F32)).astype(F32)
    u = (F32(a) * x).astype(F32)
    w = (F32(b) * d).astype(F32)
    return (u - w).astype(F32), x0


def dpmpp_2m_sample(vel_fn, x, sigmas):
    """A whole DPM++ 2M loop in float64 with velocity vel_fn(x, sigma) (the
    method itself, for its convergence pins)."""
    x = np.asarray(x, dtype=np.float64)
    x0_prev, s_prev = None, None
    for i in range(len(sigmas) - 1):
        s_cur, s_next = float(sigmas[i]), float(sigmas[i + 1])
        a, b, c1, c2, order = dpmpp_2m_coeffs(s_prev, s_cur, s_next)
        x0 = x - s_cur * vel_fn(x, s_cur)
        d = x0 if order == 1 else c1 * x0 - c2 * x0_prev
        x = a * x - b * d
        x0_prev, s_prev = x0, s_cur
    return x


def fbc_new_state() -> dict:
    """Empty first-block-cache state (reading S21)."""
    return {"valid": False, "r0": None, "rem": None, "steps": 0, "skipped": 0, "last_change": math.inf}


def first_block_cache_step(sw: dict, blocks, img_tokens, t: float, img_cos, img_sin, heads: int,
                           kv_cache, state: dict, threshold: float, dtype=np.float64):
    """An image-only step with the first-block cache ([MLX] "Optional
    modes", Fast mode), reading S21.  blocks: a list of block weights;
    kv_cache: the captured text K/V per block; state: fbc_new_state(),
    updated in place.  Returns vel [N, 64]."""
    H = sw["w_img"].shape[0]
    m_txt, m_img = modulation_rows(sw["w_mod"], sw["b_mod"], t, H, dtype)
    x0 = embed(sw, img_tokens, None, dtype)
    x1, _ = dit_block(x0, 0, blocks[0], m_txt, m_img, img_cos, img_sin, heads, kv_cache[0])
    r0 = x1 - x0
    change = math.inf
    if state["valid"]:
        den = float(np.sum(np.abs(state["r0"])))
        if den > 0.0:
            change = float(np.sum(np.abs(r0 - state["r0"]))) / den
    skip = change < threshold
    if skip:
        x = x1 + state["rem"]
    else:
        x = x1
        for b in range(1, len(blocks)):
            x, _ = dit_block(x, 0, blocks[b], m_txt, m_img, img_cos, img_sin, heads, kv_cache[b])
        state.update(valid=True, r0=r0, rem=x - x1)
    state["steps"] += 1
    state["skipped"] += int(skip)
    state["last_change"] = change
    return head(sw, x)


def cfg_combine(pos: np.ndarray, neg: np.ndarray, g) -> np.ndarray:
    """True-CFG prediction ([MLX] "Optional modes"), reading S20:
    neg + g * (pos - neg), each operation rounded to fp32 in that order."""
    pos = pos.astype(F32)
    neg = neg.astype(F32)
    d = (pos - neg).astype(F32)
    gd = (F32(g) * d).astype(F32)
    return (neg + gd).astype(F32)


def euler_update_cfg(x: np.ndarray, pos: np.ndarray, neg: np.ndarray, g, sigma_cur, sigma_next) -> np.ndarray:
    """The S14 Euler update on the S20 guided prediction."""
    return euler_update(x, cfg_combine(pos, neg, g), sigma_cur, sigma_next)


# ------------------------------------------------------------------ metrics

def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    """||a - ref||_2 / ||ref||_2 over all elements (reading S13)."""
    a = a.astype(np.float64)
    ref = ref.astype(np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def min_token_corr(a: np.ndarray, ref: np.ndarray) -> float:
    """Minimum over tokens of the Pearson correlation over each token's 64
    channels (reading S13)."""
    a = a.astype(np.float64)
    ref = ref.astype(np.float64)
    a = a - a.mean(axis=1, keepdims=True)
    r = ref - ref.mean(axis=1, keepdims=True)
    num = np.sum(a * r, axis=1)
    den = np.sqrt(np.sum(a * a, axis=1) * np.sum(r * r, axis=1))
    return float(np.min(num / den))
