"""GPU parity of the text encoder (the Qwen3-VL-8B text stack of the port
page's pieces table; bf16 weights, fp32 compute):

  - the reduced stack (hidden 512, GQA 4:1, 2 layers, L 24) and the full-width
    stack with 2 layers (hidden 4096, GQA 32:8, the pages' oracle length 32,
    the printed system-prefix ids) against the float64 oracle: relative L2 and
    the per-token correlation gate of the page's fp32-compute paragraph;
  - the full 36-layer stack against the oracle at L 64, and causality at full
    depth: the first 64 outputs of the L 421 forward (the 1024^2 prompt) equal
    the L 64 forward bit for bit;
  - an id outside the vocabulary gives a NaN row (and nothing else changes).

Bars: fp32 arithmetic through the 3-plane bf16 split (exact products, fp32
sums) puts the forward within ~1e-6 of float64; the bars leave two orders of
magnitude: rel L2 <= 1e-4 and every token's correlation >= 1 - 1e-7."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import encoder as enc
from tests.gpu_util import assert_bits_equal, host, log

pytestmark = pytest.mark.gpu

REL_BAR = 1e-4
CORR_BAR = 1.0 - 1e-7


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class Enc:
    def __init__(self, ew, keep_bits=True):
        import concurrent.futures as cf
        self.ew = ew
        self.dims = qi.make_enc_dims(ew.hidden, ew.heads, ew.kv_heads, ew.ffn, ew.n_layers, ew.vocab)
        self.embed_bits = qs.enc_embed(ew)
        with cf.ThreadPoolExecutor(8) as ex:
            self.layer_bits = list(ex.map(lambda i: qs.enc_layer_weights(ew, i, threads=1), range(ew.n_layers)))
        self.model = qi.DeviceEncoder(self.dims, self.embed_bits, self.layer_bits)

    def run(self, ids):
        import torch
        L = len(ids)
        c, s = qi.enc_rope_table(L, self.ew.rope_theta)
        out = torch.empty((L, self.ew.hidden), dtype=torch.float32, device="cuda")
        ws = qi.EncWorkspace(self.dims, L)
        qi.text_encoder_fwd(self.model, _dev(ids.astype(np.int32)), L, _dev(c), _dev(s), out, ws)
        return host(out).copy()

    def oracle(self, ids):
        emb = qs.bf16_bits_to_f32(self.embed_bits)
        layers = (qs.weights_as_f32(lb) for lb in self.layer_bits)
        c, s = enc.rope_table(len(ids), theta=self.ew.rope_theta)
        return enc.text_encoder(emb, layers, ids, c, s, self.ew.heads, self.ew.kv_heads)


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), what
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    corr = enc.min_token_corr(got, ref)
    log(f"  {what}: rel_l2={rel:.3e} min_token_corr=1-{1 - corr:.2e}")
    assert rel <= REL_BAR and corr >= CORR_BAR, (what, rel, corr)


@pytest.mark.parametrize("ew_id", [1, 2])
def test_encoder_matches_oracle(ew_id):
    ew = qs.enc_workload(ew_id)
    e = Enc(ew)
    ids = qs.enc_input_ids(ew)
    got = e.run(ids)
    _check(got, e.oracle(ids), f"{ew.name}")
    # causality: a prefix's outputs are the first rows, bit for bit
    assert_bits_equal(e.run(ids[:13]), got[:13], "prefix of 13 tokens")
    # an id outside the vocabulary: NaN row there, the causal prefix unchanged
    bad = ids.copy()
    bad[-1] = ew.vocab
    gb = e.run(bad)
    assert np.all(np.isnan(gb[-1])) and np.all(np.isfinite(gb[:-1]))
    assert_bits_equal(gb[:-1], got[:-1], "rows before the bad id")


@pytest.mark.timeout(900)
def test_encoder36_full_depth():
    ew = qs.enc_workload(3)
    log(f"{ew.name}: generating {ew.n_layers} layers")
    e = Enc(ew)
    ids = qs.enc_input_ids(ew)
    full = e.run(ids)
    assert np.all(np.isfinite(full))
    short = e.run(ids[:64])
    assert_bits_equal(full[:64], short, "first 64 of L 421 vs L 64")
    log("  oracle, 36 layers at L 64")
    _check(short, e.oracle(ids[:64]), "enc36 L64")
