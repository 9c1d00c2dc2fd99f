"""Pins of the text-encoder oracle (CPU only).

What fixes them:
  - an independent implementation of the same architecture: the Qwen3-VL
    text model of the transformers library, in float64 with the same weights
    and the same RoPE rows, whose last decoder layer's output (taken with a
    forward hook, before the final norm, as [PORT] prescribes) must equal
    the oracle's hidden states to 1e-6 (the library keeps the RMSNorm
    statistics and the softmax in fp32 even in a float64 model) -- this fixes the
    readings E1-E4 (layer order, q/k norm placement, rotate-half pairs, GQA
    grouping);
  - the RoPE table of reading E3 against the library's own fp32 RoPE rows;
  - closed forms: position 0 leaves q, k unrotated; the rotation keeps each
    pair's norm; causality (appending tokens leaves earlier outputs unchanged,
    [HOST] s.3);
  - planted mistakes (rotating adjacent pairs, GQA groups interleaved) fail the
    library comparison."""
import math

import numpy as np
import pytest

import qi_synth as qs
from oracle import encoder as enc
from tests.oracle_plant import planted

torch = pytest.importorskip("torch")
qwen3_vl = pytest.importorskip("transformers.models.qwen3_vl.modeling_qwen3_vl")

EW = qs.enc_workload(1)


def _weights(ew=EW):
    emb = qs.bf16_bits_to_f32(qs.enc_embed(ew))
    layers = [qs.weights_as_f32(qs.enc_layer_weights(ew, i)) for i in range(ew.n_layers)]
    return emb, layers


def _hf_model(ew, emb, layers):
    from transformers.models.qwen3_vl.configuration_qwen3_vl import Qwen3VLTextConfig
    cfg = Qwen3VLTextConfig(vocab_size=ew.vocab, hidden_size=ew.hidden, intermediate_size=ew.ffn,
                            num_hidden_layers=ew.n_layers, num_attention_heads=ew.heads,
                            num_key_value_heads=ew.kv_heads, head_dim=ew.head_dim, rms_norm_eps=1e-6,
                            rope_parameters={"rope_type": "default", "rope_theta": ew.rope_theta,
                                             "mrope_section": [24, 20, 20], "mrope_interleaved": True},
                            attention_bias=False)
    cfg._attn_implementation = "eager"
    m = qwen3_vl.Qwen3VLTextModel(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    with torch.no_grad():
        m.embed_tokens.weight.copy_(t(emb))
        for lyr, lw in zip(m.layers, layers):
            a = lyr.self_attn
            a.q_proj.weight.copy_(t(lw["w_q"]))
            a.k_proj.weight.copy_(t(lw["w_k"]))
            a.v_proj.weight.copy_(t(lw["w_v"]))
            a.o_proj.weight.copy_(t(lw["w_o"]))
            a.q_norm.weight.copy_(t(lw["q_norm"]))
            a.k_norm.weight.copy_(t(lw["k_norm"]))
            lyr.mlp.gate_proj.weight.copy_(t(lw["w_gate"]))
            lyr.mlp.up_proj.weight.copy_(t(lw["w_up"]))
            lyr.mlp.down_proj.weight.copy_(t(lw["w_down"]))
            lyr.input_layernorm.weight.copy_(t(lw["in_norm"]))
            lyr.post_attention_layernorm.weight.copy_(t(lw["post_norm"]))
    return m


def _hf_run(m, ids):
    out = {}
    h = m.layers[-1].register_forward_hook(lambda mod, inp, o: out.__setitem__("h", o[0] if isinstance(o, tuple) else o))
    with torch.no_grad():
        ii = torch.from_numpy(ids.astype(np.int64))[None]
        pos = torch.arange(len(ids))[None]
        cos, sin = m.rotary_emb(m.embed_tokens(ii), pos)
        m(input_ids=ii)
    h.remove()
    # the library's rows duplicate each frequency over the two halves
    return out["h"][0].numpy(), cos[0, :, :64].numpy(), sin[0, :, :64].numpy()


def test_matches_the_library_model():
    emb, layers = _weights()
    ids = qs.enc_input_ids(EW)
    ref, cos, sin = _hf_run(_hf_model(EW, emb, layers), ids)
    got = enc.text_encoder(emb, layers, ids, cos, sin, EW.heads, EW.kv_heads)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 1e-6, err


def test_rope_table_matches_the_library_rows():
    emb, layers = _weights()
    _, cos, sin = _hf_run(_hf_model(EW, emb, layers), qs.enc_input_ids(EW))
    c, s = enc.rope_table(EW.L_full)
    assert np.abs(c - cos).max() < 2e-6 and np.abs(s - sin).max() < 2e-6
    assert np.array_equal(c[0], np.ones(64, np.float32)) and np.array_equal(s[0], np.zeros(64, np.float32))


def test_rotation_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 10, 128))
    cos, sin = enc.rope_table(10)
    y = enc.rope_rotate_half(x, cos.astype(np.float64), sin.astype(np.float64))
    assert np.allclose(y[:, 0], x[:, 0], atol=0)                              # position 0: identity
    n_x = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_y = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n_x, n_y, rtol=1e-6)                                   # each pair keeps its norm


def test_causal():
    emb, layers = _weights()
    ids = qs.enc_input_ids(EW)
    cos, sin = enc.rope_table(EW.L_full)
    full = enc.text_encoder(emb, layers, ids, cos, sin, EW.heads, EW.kv_heads)
    part = enc.text_encoder(emb, layers, ids[:13], cos[:13], sin[:13], EW.heads, EW.kv_heads)
    assert np.allclose(part, full[:13], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fn,old,new", [
    ("rope_rotate_half", "a, b = x[..., :half], x[..., half:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    ("gqa_causal_attention", "kk = np.repeat(k, group, axis=0)", "kk = np.tile(k, (group, 1, 1))"),
])
def test_planted_mistakes_fail_the_library_comparison(fn, old, new):
    wide = qs.enc_workload(1, kv_heads=2)   # two kv heads, so the grouping order matters
    emb, layers = _weights(wide)
    ids = qs.enc_input_ids(wide)
    ref, cos, sin = _hf_run(_hf_model(wide, emb, layers), ids)
    bad_fn = planted(getattr(enc, fn), old, new, module=enc)
    import inspect
    import textwrap
    ns = dict(vars(enc))
    ns[fn] = bad_fn
    for name in ("encoder_layer", "text_encoder"):
        exec(compile(textwrap.dedent(inspect.getsource(getattr(enc, name))), "<planted>", "exec"), ns)
    got = ns["text_encoder"](emb, layers, ids, cos, sin, wide.heads, wide.kv_heads)
    good = enc.text_encoder(emb, layers, ids, cos, sin, wide.heads, wide.kv_heads)
    assert np.abs(good - ref).max() / np.abs(ref).max() < 1e-6
    assert np.abs(got - ref).max() / np.abs(ref).max() > 1e-3


def test_library_host_rope_rows_equal_the_oracle():
    """The library's host RoPE rows (qi_enc_rope_table) are bit-identical to
    the oracle's reading-E3 table (host logic, no GPU)."""
    import block_causal_attention_qi_amd as qi
    for L in (1, 32, 421, 512):
        c, s = qi.enc_rope_table(L)
        oc, os_ = enc.rope_table(L)
        assert np.array_equal(c, oc) and np.array_equal(s, os_)
