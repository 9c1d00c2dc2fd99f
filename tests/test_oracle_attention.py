"""Pins of the oracle's block-causal attention (CPU only).

What fixes it: the port page's DiT row (attention as two SDPA calls, text->text
causal and image->all, "the reference's own segment decomposition, so no mask
input") and the MLX page's "Text K/V reuse" (text rows never see the image).
The decomposition must equal ONE masked softmax over [text | image] keys with
the block-causal mask; the single-mask version is written as brute-force loops
and checked against torch's SDPA."""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import dit


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _allowed(i, j, L):
    """Block-causal mask of the pages: a text query i (< L) sees text keys
    j <= i; an image query sees every key."""
    if i < L:
        return j < L and j <= i
    return True


def _brute_force(q, k, v, L):
    heads, T, d = q.shape
    out = np.zeros_like(q)
    for h in range(heads):
        for i in range(T):
            js = [j for j in range(T) if _allowed(i, j, L)]
            sc = [sum(q[h, i, c] * k[h, j, c] for c in range(d)) / math.sqrt(d) for j in js]
            mx = max(sc)
            ws = [math.exp(s - mx) for s in sc]
            tot = sum(ws)
            for c in range(d):
                out[h, i, c] = sum(w * v[h, j, c] for w, j in zip(ws, js)) / tot
    return out


def _decomp(q, k, v, L):
    o_t, o_i = dit.block_causal_attention(q[:, :L], k[:, :L], v[:, :L], q[:, L:], k[:, L:], v[:, L:])
    return np.concatenate([o_t, o_i], axis=1)


def test_decomposition_equals_single_masked_softmax():
    L, N, d, heads = 3, 5, 8, 2
    q, k, v = (_rand((heads, L + N, d), s) for s in (1, 2, 3))
    got = _decomp(q, k, v, L)
    ref = _brute_force(q, k, v, L)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_decomposition_matches_torch_sdpa_with_mask():
    L, N, d, heads = 7, 13, 128, 3
    q, k, v = (_rand((heads, L + N, d), s) for s in (4, 5, 6))
    T = L + N
    mask = torch.tensor([[_allowed(i, j, L) for j in range(T)] for i in range(T)])
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v)), attn_mask=mask).numpy()
    assert np.max(np.abs(_decomp(q, k, v, L) - ref)) < 1e-12


def test_segments_match_torch_sdpa():
    L, N, d, heads = 6, 10, 128, 2
    q, k, v = (_rand((heads, L + N, d), s) for s in (7, 8, 9))
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    ref_txt = F.scaled_dot_product_attention(tq[:, :L], tk[:, :L], tv[:, :L], is_causal=True).numpy()
    ref_img = F.scaled_dot_product_attention(tq[:, L:], tk, tv).numpy()
    o_t, o_i = dit.block_causal_attention(q[:, :L], k[:, :L], v[:, :L], q[:, L:], k[:, L:], v[:, L:])
    assert np.max(np.abs(o_t - ref_txt)) < 1e-12
    assert np.max(np.abs(o_i - ref_img)) < 1e-12


def test_text_rows_ignore_image_keys():
    L, N, d, heads = 4, 6, 16, 1
    q, k, v = (_rand((heads, L + N, d), s) for s in (10, 11, 12))
    a = _decomp(q, k, v, L)
    k2, v2 = k.copy(), v.copy()
    k2[:, L:] += 3.0
    v2[:, L:] -= 5.0
    b = _decomp(q, k2, v2, L)
    assert np.array_equal(a[:, :L], b[:, :L])
    assert not np.allclose(a[:, L:], b[:, L:])


def test_negative_control_causal_image_rows():
    """Making the image rows causal (a plausible mistake) must break the
    brute-force pin."""
    L, N, d, heads = 3, 5, 8, 1
    q, k, v = (_rand((heads, L + N, d), s) for s in (13, 14, 15))
    ref = _brute_force(q, k, v, L)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    wrong = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
    assert np.max(np.abs(wrong[:, L:] - ref[:, L:])) > 1e-3


def test_sdpa_scale_is_inverse_sqrt_d():
    # one query, two keys, v = identity columns: weights are softmax(qk/sqrt(d))
    d = 128
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 2.0
    k = np.zeros((1, 2, d)); k[0, 0, 0] = 3.0
    v = np.zeros((1, 2, d)); v[0, 0, 0] = 1.0; v[0, 1, 1] = 1.0
    o = dit.sdpa(q, k, v, causal=False)
    s0 = 6.0 / math.sqrt(d)
    w0 = math.exp(s0) / (math.exp(s0) + 1.0)
    assert abs(o[0, 0, 0] - w0) < 1e-15 and abs(o[0, 0, 1] - (1 - w0)) < 1e-15
