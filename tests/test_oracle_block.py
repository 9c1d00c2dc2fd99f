"""Pins of the oracle's block wiring, modulation, embed/head and reuse
exactness (CPU only).

What fixes them: library routines (torch's rms_norm, silu, SDPA with an
explicit block-causal mask, complex RoPE) on special cases where a reading
reduces to a plain pre-norm transformer block; closed forms (zero gates give
an identity block; the t = 0 embedding is [1..1 | 0..0]); and the invariants
the MLX page states for text-K/V reuse (text rows never see the image, so
their K/V do not depend on the image tokens, t or N, and a cached step equals
full recompute)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import qi_synth as qs
from oracle import dit
from tests.oracle_plant import planted, planted_step, step_with

WL = qs.workload(1)


def _weights(wl=WL):
    sw = qs.shared_weights(wl, as_bf16=False)
    bw = qs.block_weights(wl, 0, as_bf16=False)
    return sw, bw


def _rows(wl=WL, L=None):
    return dit.rope_rows(wl.L if L is None else L, wl.h, wl.w)


def test_rms_norm_matches_torch():
    x = np.random.default_rng(0).standard_normal((7, 512))
    g = 1 + 0.02 * np.random.default_rng(1).standard_normal(512)
    ref = F.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.max(np.abs(dit.rms_norm(x, g) - ref)) < 1e-13


def test_zero_center_norm_matches_torch():
    x = np.random.default_rng(2).standard_normal((3, 64))
    w = 0.02 * np.random.default_rng(3).standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(1 + w), eps=1e-6).numpy()
    assert np.max(np.abs(dit.zero_center_rms_norm(x, w) - ref)) < 1e-13


def test_silu_matches_torch():
    u = np.linspace(-30, 30, 1001)
    assert np.max(np.abs(dit.silu(u) - F.silu(torch.from_numpy(u)).numpy())) < 1e-13


def test_timestep_embedding_closed_forms():
    H = 512
    e0 = dit.timestep_embedding(0.0, H)
    assert np.all(e0[:H // 2] == 1.0) and np.all(e0[H // 2:] == 0.0)
    e = dit.timestep_embedding(0.7, H)
    assert abs(e[0] - np.cos(700.0)) < 1e-15 and abs(e[H // 2] - np.sin(700.0)) < 1e-15
    # last frequency 10000^(-(H/2-1)/(H/2))
    f = 10000.0 ** (-(H // 2 - 1) / (H // 2))
    assert abs(e[H - 1] - np.sin(700.0 * f)) < 1e-15


def test_modulation_t0_row_closed_form():
    sw, _ = _weights()
    H = WL.hidden
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], 0.7, H)
    ref = sw["w_mod"].astype(np.float64)[:, :H // 2].sum(axis=1) + sw["b_mod"]
    assert np.max(np.abs(m_txt - ref)) < 1e-12
    assert m_txt.shape == (4 * H,) and not np.allclose(m_txt, m_img)


def _zero_gate_weights():
    sw, bw = _weights()
    H = WL.hidden
    sw = dict(sw)
    w_mod = sw["w_mod"].copy(); b_mod = sw["b_mod"].copy()
    for chunk in (1, 3):                       # gate1, gate2 (reading S2)
        w_mod[chunk * H:(chunk + 1) * H] = 0
        b_mod[chunk * H:(chunk + 1) * H] = 0
    sw["w_mod"], sw["b_mod"] = w_mod, b_mod
    return sw, bw


def test_zero_gates_give_identity_blocks():
    sw, bw = _zero_gate_weights()
    X = qs.img_tokens(WL)
    E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    vel = dit.dit_step(sw, [bw, bw], WL.L, X, E, 0.7, tc, ts, ic, is_, WL.heads)
    # closed form: proj_out(RMSNorm(img_in(X)))
    x_img = X.astype(np.float64) @ sw["w_img"].T.astype(np.float64) + sw["b_img"]
    ref = dit.rms_norm(x_img, sw["norm_out"]) @ sw["w_out"].T.astype(np.float64) + sw["b_out"]
    assert np.max(np.abs(vel - ref)) < 1e-12


def _plain_modulation_weights():
    """scale rows 0 and gate rows 1: the block reduces to a plain pre-norm
    block (x + attn(norm x), then x + mlp(norm x))."""
    sw, bw = _weights()
    H = WL.hidden
    sw = dict(sw)
    w_mod = sw["w_mod"].copy(); b_mod = sw["b_mod"].copy()
    w_mod[:] = 0
    b_mod[:] = 0
    b_mod[H:2 * H] = 1.0
    b_mod[3 * H:4 * H] = 1.0
    sw["w_mod"], sw["b_mod"] = w_mod, b_mod
    return sw, bw


def _torch_plain_block(x, L, bw, cos, sin, heads):
    """Library-built pre-norm block: torch rms_norm, complex RoPE, one SDPA
    call with the explicit block-causal boolean mask, silu."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    X = t(x)
    T, H = X.shape
    h = F.rms_norm(X, (H,), t(bw["norm1"]), eps=1e-6)
    qkv = h @ t(bw["w_qkv"]).T
    q, k, v = (qkv[:, i * H:(i + 1) * H].reshape(T, heads, 64, 2) for i in range(3))
    rot = torch.complex(t(cos), t(sin))[:, None, :]
    q = torch.view_as_real(torch.view_as_complex(q.contiguous()) * rot).reshape(T, heads, 128)
    k = torch.view_as_real(torch.view_as_complex(k.contiguous()) * rot).reshape(T, heads, 128)
    v = v.reshape(T, heads, 128)
    idx = torch.arange(T)
    mask = (idx[None, :] <= idx[:, None]) & (idx[None, :] < L)
    mask = mask | (idx[:, None] >= L)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), attn_mask=mask)
    o = o.transpose(0, 1).reshape(T, H)
    X = X + o @ t(bw["w_o"]).T
    h2 = F.rms_norm(X, (H,), t(bw["norm2"]), eps=1e-6)
    u = h2 @ t(bw["w_gu"]).T
    Fh = u.shape[1] // 2
    X = X + (F.silu(u[:, :Fh]) * u[:, Fh:]) @ t(bw["w_down"]).T
    return X.numpy()


def test_plain_block_matches_torch_library_block():
    sw, bw = _plain_modulation_weights()
    X = qs.img_tokens(WL)
    E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], 0.7, WL.hidden)
    x0 = dit.embed(sw, X, E)
    cos, sin = np.concatenate([tc, ic]), np.concatenate([ts, is_])
    got, _ = dit.dit_block(x0, WL.L, bw, m_txt, m_img, cos, sin, WL.heads)
    ref = _torch_plain_block(x0, WL.L, bw, cos, sin, WL.heads)
    assert np.max(np.abs(got - ref)) < 1e-10 * max(1.0, np.max(np.abs(ref)))


def test_negative_control_scale_without_one_fails_plain_block():
    sw, bw = _plain_modulation_weights()
    blk = planted(dit.dit_block, "(1.0 + s1)", "s1")
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], 0.7, WL.hidden)
    x0 = dit.embed(sw, X, E)
    cos, sin = np.concatenate([tc, ic]), np.concatenate([ts, is_])
    got, _ = blk(x0, WL.L, bw, m_txt, m_img, cos, sin, WL.heads)
    ref = _torch_plain_block(x0, WL.L, bw, cos, sin, WL.heads)
    assert np.max(np.abs(got - ref)) > 1e-3


def _step(sw, bws, X, E, t, L=None, kv=None, capture=False, step=dit.dit_step, return_x=False, wl=WL):
    L = wl.L if L is None else L
    tc, ts, ic, is_ = dit.rope_rows(L, wl.h, wl.w) if X.shape[0] == wl.N else dit.rope_rows(L, 1, X.shape[0])
    return step(sw, bws, L, X, E, t, tc, ts, ic, is_, wl.heads, kv_cache=kv, capture=capture, return_x=return_x)


def test_text_rows_invariant_to_image_and_t():
    sw, bw = _weights()
    bws = [bw, qs.block_weights(WL, 1, as_bf16=False)]
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    (v1, c1), x1 = _step(sw, bws, X, E, 0.7, capture=True, return_x=True)
    X2 = qs.img_tokens(WL, seed=99)
    (v2, c2), x2 = _step(sw, bws, X2, E, 0.3, capture=True, return_x=True)
    assert np.array_equal(x1[:WL.L], x2[:WL.L])                       # bit-exact, same shapes
    for (k1, vv1), (k2, vv2) in zip(c1, c2):
        assert np.array_equal(k1, k2) and np.array_equal(vv1, vv2)
    assert not np.allclose(v1, v2)
    # a different N (other grid): text K/V equal up to BLAS blocking
    X3 = qs.noise_latent(4, 4, seed=5)
    (v3, c3), x3 = _step(sw, bws, X3, E, 0.5, capture=True, return_x=True)
    for (k1, vv1), (k3, vv3) in zip(c1, c3):
        assert np.max(np.abs(k1 - k3)) < 1e-12 and np.max(np.abs(vv1 - vv3)) < 1e-12


def test_negative_control_text_rows_with_sampled_t_break_invariance():
    sw, bw = _weights()
    step = planted_step("mt, mi = split_mod(m_txt.astype(dt), H), split_mod(m_img.astype(dt), H)",
                        "mt, mi = split_mod(m_img.astype(dt), H), split_mod(m_img.astype(dt), H)")
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    (_, c1) = _step(sw, [bw], X, E, 0.7, capture=True, step=step)
    (_, c2) = _step(sw, [bw], X, E, 0.3, capture=True, step=step)
    assert not np.array_equal(c1[0][0], c2[0][0])


def test_cached_step_equals_full_recompute():
    sw, bw = _weights()
    bws = [bw, qs.block_weights(WL, 1, as_bf16=False)]
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    _, cache = _step(sw, bws, X, E, 0.9, capture=True)
    X2 = qs.img_tokens(WL, seed=7)
    full = _step(sw, bws, X2, E, 0.45)
    cached = _step(sw, bws, X2, None, 0.45, kv=cache)
    assert np.max(np.abs(full - cached)) < 1e-12 * np.max(np.abs(full))


def test_negative_control_causal_image_rows_move_vel():
    """Image rows made causal over the image only (a plausible mistake) must
    move vel well past the 2e-2 bar."""
    sw, bw = _weights()
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    good = _step(sw, [bw], X, E, 0.6)
    bad_attn = planted(dit.block_causal_attention,
                       "o_img = sdpa(q_img, k_all, v_all, causal=False, bf16=bf16)",
                       "o_img = sdpa(q_img, k_img, v_img, causal=True, bf16=bf16)")
    bad = _step(sw, [bw], X, E, 0.6, step=step_with(block_causal_attention=bad_attn))
    assert dit.rel_l2(bad, good) > 2e-2


def test_metrics():
    a = np.random.default_rng(0).standard_normal((10, 64))
    assert dit.rel_l2(a, a) == 0.0 and abs(dit.min_token_corr(a, a) - 1.0) < 1e-12
    b = a.copy(); b[3] = -b[3]
    assert dit.min_token_corr(b, a) < -0.99
    assert abs(dit.rel_l2(2 * a, a) - 1.0) < 1e-12


def test_block_rows_equals_full_block():
    """The row-sampled block (used for parity at full sizes) is the full block
    restricted to the chosen rows, joint and image-only."""
    sw, bw = _weights()
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    m_txt, m_img = dit.modulation_rows(sw["w_mod"], sw["b_mod"], 0.7, WL.hidden)
    x0 = dit.embed(sw, X, E)
    cos, sin = np.concatenate([tc, ic]), np.concatenate([ts, is_])
    full, kv = dit.dit_block(x0, WL.L, bw, m_txt, m_img, cos, sin, WL.heads)
    rows = [0, 3, WL.L - 1, WL.L, WL.L + 17, WL.L + WL.N - 1]
    part = dit.dit_block_rows(x0, WL.L, bw, m_txt, m_img, cos, sin, WL.heads, rows)
    assert np.max(np.abs(part - full[rows])) < 1e-12 * np.max(np.abs(full))
    fi, _ = dit.dit_block(x0[WL.L:], 0, bw, m_txt, m_img, ic, is_, WL.heads, kv_text=kv)
    pi = dit.dit_block_rows(x0[WL.L:], 0, bw, m_txt, m_img, ic, is_, WL.heads, [0, 5, WL.N - 1], kv_text=kv)
    assert np.max(np.abs(pi - fi[[0, 5, WL.N - 1]])) < 1e-12 * np.max(np.abs(fi))


def test_round_bf16_closed_forms():
    r = dit.round_bf16
    one = np.float64(1.0)
    assert r(np.array([one]))[0] == 1.0
    assert r(np.array([1 + 2.0 ** -8]))[0] == 1.0                 # tie -> even mantissa
    assert r(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6    # tie -> even mantissa
    assert r(np.array([1 + 2.0 ** -8 + 2.0 ** -20]))[0] == 1 + 2.0 ** -7
    assert r(np.array([-3.0]))[0] == -3.0 and r(np.array([0.0]))[0] == 0.0
    x = np.random.default_rng(0).standard_normal(10000)
    y = r(x)
    assert np.max(np.abs(y - x) / np.abs(x)) <= 2.0 ** -8
    assert np.array_equal(r(y), y)


def test_bf16_mode_stays_within_the_rounding_envelope():
    """One block in the bf16-compute reading differs from the exact block by
    more than round-off of fp64 and less than the bf16 band."""
    sw, bw = _weights()
    X = qs.img_tokens(WL); E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    exact = dit.dit_step(sw, [bw], WL.L, X, E, 0.7, tc, ts, ic, is_, WL.heads)
    b16 = dit.dit_step(sw, [bw], WL.L, X, E, 0.7, tc, ts, ic, is_, WL.heads, bf16=True)
    rel = dit.rel_l2(b16, exact)
    assert 1e-4 < rel < 1e-2, rel


def _structured_shared(wl=WL):
    """Shared weights whose projections are selections with a known product:
    W_txt a cyclic shift (row j reads feature j - 1: not symmetric, so a
    transposed W_txt lands every value two features off), W_img and W_out
    scatter / gather matrices, and distinct biases and norm weights (so a
    dropped bias or norm weight changes the result)."""
    sw, bw = _weights(wl)
    H, D = wl.hidden, wl.txt_dim
    sw = dict(sw)
    w_txt = np.zeros((H, D), np.float32)
    w_txt[(np.arange(D) + 1) % H, np.arange(D)] = 1.0
    w_img = np.zeros((H, 64), np.float32)
    w_img[5 * np.arange(64) + 2, np.arange(64)] = 1.0
    w_out = np.zeros((64, H), np.float32)
    w_out[np.arange(64), 7 * np.arange(64) + 3] = 1.0
    sw.update(w_txt=w_txt, b_txt=(100.0 + np.arange(H)).astype(np.float32),
              txt_norm=(0.25 + 0.5 * (np.arange(D) % 3)).astype(np.float32),
              w_img=w_img, b_img=(-50.0 - np.arange(H)).astype(np.float32),
              w_out=w_out, b_out=(1000.0 + np.arange(64)).astype(np.float32),
              norm_out=(1.0 + 0.01 * np.arange(H)).astype(np.float32))
    return sw, bw


def test_text_projection_and_img_in_closed_form():
    """embed() on one-hot text rows c * e_i: the zero-centred norm gives
    c / sqrt(c^2/D + eps) * (1 + w_i) at feature i, the cyclic-shift W_txt
    moves it to feature i + 1, and b_txt adds its own value everywhere; the
    image rows are X scattered to features 5c + 2 plus b_img.  Fails for a
    transposed W_txt, a dropped b_txt or norm weight, or a transposed W_img."""
    sw, _ = _structured_shared()
    H, D = WL.hidden, WL.txt_dim
    idx = np.array([0, 3, 100, D - 1, 257, 31, 64, 9])[:WL.L]
    c = np.array([1.0, -2.0, 0.5, 3.0, -1.5, 10.0, 0.25, -4.0])[:WL.L]
    E = np.zeros((WL.L, D), np.float32)
    E[np.arange(WL.L), idx] = c
    X = qs.img_tokens(WL)
    x = dit.embed(sw, X, E)
    ref_txt = np.tile(100.0 + np.arange(H), (WL.L, 1))
    wn = 0.25 + 0.5 * (idx % 3)
    ref_txt[np.arange(WL.L), (idx + 1) % H] += c / np.sqrt(c * c / D + 1e-6) * (1.0 + wn)
    ref_img = np.tile(-50.0 - np.arange(H), (WL.N, 1))
    ref_img[:, 5 * np.arange(64) + 2] += X
    assert x.shape == (WL.L + WL.N, H)
    assert np.max(np.abs(x[:WL.L] - ref_txt)) < 1e-9
    assert np.max(np.abs(x[WL.L:] - ref_img)) < 1e-9


def test_head_closed_form_on_the_image_rows():
    """A step whose gates are zero leaves x = embed(); the gather W_out then
    reads feature 7c + 3 of each IMAGE row, divided by the row's RMS (over all
    H features, eps 1e-6), times norm_out at that feature, plus b_out[c].  The
    reference below is that closed form written from X alone: it fails if
    the head reads the text rows, drops norm_out or b_out, or normalises
    over the wrong axis."""
    sw, bw = _structured_shared()
    H = WL.hidden
    for chunk in (1, 3):                        # zero gates (reading S2)
        sw["w_mod"] = sw["w_mod"].copy(); sw["b_mod"] = sw["b_mod"].copy()
        sw["w_mod"][chunk * H:(chunk + 1) * H] = 0
        sw["b_mod"][chunk * H:(chunk + 1) * H] = 0
    X = qs.img_tokens(WL).astype(np.float64)
    E = qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    vel = dit.dit_step(sw, [bw], WL.L, X.astype(np.float32), E, 0.7, tc, ts, ic, is_, WL.heads)
    # image row r of x: b_img = -50 - j everywhere, plus X[r, c] at feature 5c + 2
    j = np.arange(H)
    x_img = np.tile(-50.0 - j, (WL.N, 1))
    x_img[:, 5 * np.arange(64) + 2] += X
    inv_rms = 1.0 / np.sqrt(np.mean(x_img * x_img, axis=1) + 1e-6)
    f = 7 * np.arange(64) + 3
    g = (1.0 + 0.01 * f).astype(np.float32).astype(np.float64)       # norm_out as stored (fp32)
    ref = x_img[:, f] * inv_rms[:, None] * g[None, :] + (1000.0 + np.arange(64))[None, :]
    assert np.max(np.abs(vel - ref)) < 1e-9


@pytest.mark.parametrize("old,new", [
    ('sw["w_txt"].astype(dtype).T', 'sw["w_txt"].astype(dtype)'),                 # transposed W_txt
    (' + sw["b_txt"].astype(dtype)', ''),                                          # dropped b_txt
    ('zero_center_rms_norm(txt_feats.astype(dtype), sw["txt_norm"])',
     'rms_norm(txt_feats.astype(dtype), sw["txt_norm"])'),                         # weight not zero-centred
    ('sw["w_img"].astype(dtype).T', 'sw["w_img"].astype(dtype).T[:, ::-1]'),       # features reversed
])
def test_negative_controls_break_the_text_projection_pin(old, new):
    bad = planted(dit.embed, old, new)
    sw, _ = _structured_shared()
    D = WL.txt_dim
    E = np.zeros((WL.L, D), np.float32)
    E[np.arange(WL.L), np.arange(WL.L) * 3] = 2.0
    X = qs.img_tokens(WL)
    good = dit.embed(sw, X, E)
    assert np.max(np.abs(bad(sw, X, E) - good)) > 1e-3


@pytest.mark.parametrize("plant", ["text rows", "no norm_out", "no b_out"])
def test_negative_controls_break_the_head_pin(plant):
    sw, bw = _structured_shared()
    H = WL.hidden
    for chunk in (1, 3):
        sw["w_mod"] = sw["w_mod"].copy(); sw["b_mod"] = sw["b_mod"].copy()
        sw["w_mod"][chunk * H:(chunk + 1) * H] = 0
        sw["b_mod"][chunk * H:(chunk + 1) * H] = 0
    X, E = qs.img_tokens(WL), qs.txt_feats(WL)
    tc, ts, ic, is_ = _rows()
    args = (sw, [bw], WL.L, X, E, 0.7, tc, ts, ic, is_, WL.heads)
    good = dit.dit_step(*args)
    if plant == "text rows":
        step = planted(dit.dit_step, "vel = head(sw, x[L_rows:])", "vel = head(sw, x[:x.shape[0] - L_rows])")
    else:
        old = 'rms_norm(x_img, sw["norm_out"])' if plant == "no norm_out" else ' + sw["b_out"].astype(dt)'
        new = 'rms_norm(x_img, np.ones_like(sw["norm_out"]))' if plant == "no norm_out" else ''
        step = step_with(head=planted(dit.head, old, new))
    assert np.max(np.abs(step(*args) - good)) > 1e-3
