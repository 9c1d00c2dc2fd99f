"""GPU parity of the HIP components through the C ABI: the bf16 MFMA GEMM, the
block-causal attention kernel, the shared modulation GEMV and the fp32 Euler
update, each against a plain CPU computation of the same operation on the
same bf16/fp32 input values (the oracle's functions where it has one)."""
import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
import qi_synth as qs
from oracle import dit
from tests.gpu_util import assert_bits_equal, bf16_bits, bf16_vals, host, log

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# (4096, 4096, 256), (4000, 4096, 192) and (4100, 4096, 832) run the 256 x 256
# LDS-copy kernel: K steps only in its unrolled tail (4, 3), and 13 = 2 x 6 + 1
# steps with a ragged last row tile
@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (200, 256, 192), (278, 384, 512), (1070, 512, 4096),
                                   (4096, 4096, 256), (4000, 4096, 192), (4100, 4096, 832)])
def test_linear_bf16_matches_fp64_matmul(M, N, K):
    import torch
    log(f"linear M={M} N={N} K={K}")
    a = bf16_bits(qs.normal_array((M, K), seed=1))
    w = bf16_bits(qs.normal_array((N, K), seed=2, scale=0.02))
    b = qs.normal_array((N,), seed=3, scale=0.1)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qi.linear_bf16(_dev(a), _dev(w), _dev(b), C)
    got = host(C)
    ref = bf16_vals(a) @ bf16_vals(w).T + b
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err < 2e-5, err
    # no bias
    qi.linear_bf16(_dev(a), _dev(w), None, C)
    got = host(C)
    assert np.max(np.abs(got - (ref - b))) / np.max(np.abs(ref)) < 2e-5


def test_linear_bf16_rows_do_not_depend_on_the_launch_split():
    """4100 rows go out as a 4096-row launch of 256 x 256 tiles plus a 4-row
    tail launch; inside an 8192-row product (one launch, no tail) the same rows
    must come out bit for bit the same (every element sees one MFMA sequence
    whatever the tile shape or launch)."""
    import torch
    M, N, K = 4100, 4096, 832
    a = bf16_bits(qs.normal_array((8192, K), seed=11))
    w = bf16_bits(qs.normal_array((N, K), seed=12, scale=0.02))
    b = qs.normal_array((N,), seed=13, scale=0.1)
    C1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C2 = torch.empty((8192, N), dtype=torch.float32, device="cuda")
    qi.linear_bf16(_dev(a[:M]), _dev(w), _dev(b), C1)
    qi.linear_bf16(_dev(a), _dev(w), _dev(b), C2)
    assert_bits_equal(host(C1), host(C2)[:M], "4100 rows (head + tail launches) vs inside 8192 rows")


def test_linear_bf16_past_32_bit_offsets_matches_the_lds_kernels():
    """An A operand of more than 2 GiB (65544 rows x 16384) cannot be addressed
    with the LDS-copy kernels' 32-bit buffer offsets and runs on the
    register-staged 32x32x16 kernel; its rows must equal, bit for bit, the
    same rows computed by the LDS-copy kernels from a smaller A (the first 4096
    rows on 256 x 256 tiles with the 16x16x32 MFMA, the last 300 on 128 x 128
    tiles with 32x32x16), and match an fp64 product of the bf16 operands."""
    import torch
    M, N, K = 65544, 4096, 16384
    assert M * K * 2 > 2**31
    g = torch.Generator(device="cuda").manual_seed(21)
    a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    big = torch.empty((M, N), dtype=torch.float32, device="cuda")
    qi.linear_bf16(a.view(torch.int16), w.view(torch.int16), None, big)
    rows = {"first 4096": slice(0, 4096), "last 300": slice(M - 300, M)}
    for what, sl in rows.items():
        sub = a[sl].contiguous()
        small = torch.empty((sub.shape[0], N), dtype=torch.float32, device="cuda")
        qi.linear_bf16(sub.view(torch.int16), w.view(torch.int16), None, small)
        assert_bits_equal(host(big[sl]), host(small), f"{what} rows: register-staged vs LDS-copy kernels")
    torch.cuda.synchronize()
    pick = torch.tensor([0, 1, 4095, 33000, M - 1], device="cuda")
    ref = a[pick].double().cpu() @ w.double().cpu().t()
    got = big[pick].double().cpu()
    assert float((got - ref).abs().max() / ref.abs().max()) < 2e-5
    del a, big


def _attn_inputs(heads, L, N, seed):
    q = bf16_bits(qs.normal_array((heads, L + N, 128), seed=seed))
    k = bf16_bits(qs.normal_array((heads, L + N, 128), seed=seed + 1))
    v = bf16_bits(qs.normal_array((heads, L + N, 128), seed=seed + 2))
    return q, k, v


def _vt(v_bits, Tp):
    heads, T, d = v_bits.shape
    out = np.zeros((heads, d, Tp), np.uint16)
    out[:, :, :T] = v_bits.transpose(0, 2, 1)
    # poison the padding columns: the kernel must never let them into a result
    out[:, :, T:] = 0x7FC0   # bf16 NaN
    return out


@pytest.mark.parametrize("heads,L,N", [(2, 8, 64), (2, 37, 150), (3, 130, 70), (1, 407, 300)])
def test_block_causal_attention_matches_oracle(heads, L, N):
    import torch
    log(f"attention heads={heads} L={L} N={N}")
    q, k, v = _attn_inputs(heads, L, N, seed=10 + L)
    Lp, Np = (L + 63) // 64 * 64, (N + 63) // 64 * 64
    q_t, k_t, q_i, k_i = (_dev(np.ascontiguousarray(a)) for a in (q[:, :L], k[:, :L], q[:, L:], k[:, L:]))
    vt_t, vt_i = _dev(_vt(v[:, :L], Lp)), _dev(_vt(v[:, L:], Np))
    o = torch.empty((L + N, heads * 128), dtype=torch.int16, device="cuda")
    qi.block_causal_attention(heads, L, N, qi.QI_MODE_JOINT, q_t, k_t, vt_t, q_i, k_i, vt_i, o)
    got = bf16_vals(host(o).view(np.uint16)).reshape(L + N, heads, 128).transpose(1, 0, 2)
    qv, kv, vv = bf16_vals(q), bf16_vals(k), bf16_vals(v)
    o_t, o_i = dit.block_causal_attention(qv[:, :L], kv[:, :L], vv[:, :L], qv[:, L:], kv[:, L:], vv[:, L:])
    ref = np.concatenate([o_t, o_i], axis=1)
    assert np.all(np.isfinite(got))
    rel = dit.rel_l2(got, ref)
    mx = np.max(np.abs(got - ref))
    log(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel < 1e-2 and mx < 5e-2
    # image-only pass: same image rows, bit for bit
    o2 = torch.empty((N, heads * 128), dtype=torch.int16, device="cuda")
    qi.block_causal_attention(heads, L, N, qi.QI_MODE_IMAGE_ONLY, None, k_t, vt_t, q_i, k_i, vt_i, o2)
    assert_bits_equal(host(o2), host(o)[L:], "image-only attention rows")


def test_attention_workgroup_shape_changes_no_bit():
    """2 heads at L 407, N 1100 launch 4-wave workgroups (too few 8-wave ones
    for the CUs); 64 heads launch 8-wave ones, joint and image-only.  The
    first two heads are the same inputs in both, and their output rows must be
    the same bits."""
    import torch
    L, N, H2 = 407, 1100, 64
    q, k, v = _attn_inputs(H2, L, N, seed=90)
    Lp, Np = (L + 63) // 64 * 64, (N + 63) // 64 * 64
    outs = {}
    for heads in (2, H2):
        q_t, k_t, q_i, k_i = (_dev(np.ascontiguousarray(a[:heads])) for a in (q[:, :L], k[:, :L], q[:, L:], k[:, L:]))
        vt_t, vt_i = _dev(_vt(v[:heads, :L], Lp)), _dev(_vt(v[:heads, L:], Np))
        o = torch.empty((L + N, heads * 128), dtype=torch.int16, device="cuda")
        qi.block_causal_attention(heads, L, N, qi.QI_MODE_JOINT, q_t, k_t, vt_t, q_i, k_i, vt_i, o)
        o2 = torch.empty((N, heads * 128), dtype=torch.int16, device="cuda")
        qi.block_causal_attention(heads, L, N, qi.QI_MODE_IMAGE_ONLY, None, k_t, vt_t, q_i, k_i, vt_i, o2)
        outs[heads] = (host(o)[:, :256].copy(), host(o2)[:, :256].copy())
    assert_bits_equal(outs[2][0], outs[H2][0], "joint rows, 4-wave vs 8-wave workgroups")
    assert_bits_equal(outs[2][1], outs[H2][1], "image-only rows, 4-wave vs 8-wave workgroups")


def test_attention_lazy_rescale_path():
    """Keys scaled up tile by tile along the kernel's walk (text key tiles, then
    image key tiles) make each query's running max rise past its slack of 2^8
    on most tiles, so the accumulators are rescaled while they hold earlier
    tiles' products (random unit-scale inputs never get there after the first
    tile).  The result must still match the oracle's exact softmax."""
    import torch
    heads, L, N = 2, 200, 300
    log(f"attention lazy rescale heads={heads} L={L} N={N}")
    qa = qs.normal_array((heads, L + N, 128), seed=70) * 3.0
    ka = qs.normal_array((heads, L + N, 128), seed=71)
    va = qs.normal_array((heads, L + N, 128), seed=72)
    nt_t = (L + 63) // 64
    tile = np.concatenate([np.arange(L) // 64, nt_t + np.arange(N) // 64])  # position in the walk
    ka = ka * (1.0 + tile)[None, :, None]
    q, k, v = bf16_bits(qa), bf16_bits(ka), bf16_bits(va)
    qv, kv, vv = bf16_vals(q), bf16_vals(k), bf16_vals(v)
    # the construction does what it claims: count, per image query, the tiles
    # whose max exceeds the running max by more than 8 (log2 units)
    s = np.einsum("hqd,hkd->hqk", qv[:, L:], kv) / np.sqrt(128.0) * np.log2(np.e)
    tmax = np.stack([s[:, :, tile == j].max(axis=2) for j in range(int(tile.max()) + 1)], axis=2)
    run = tmax[:, :, 0].copy()
    raises = np.zeros(run.shape, int)
    for j in range(1, tmax.shape[2]):
        up = tmax[:, :, j] > run + 8.0
        raises += up
        run = np.where(up, tmax[:, :, j], run)
    log(f"  rescales after the first tile per image query: mean {raises.mean():.2f}, min {raises.min()}")
    assert raises.mean() >= 3 and raises.min() >= 1
    Lp, Np = (L + 63) // 64 * 64, (N + 63) // 64 * 64
    q_t, k_t, q_i, k_i = (_dev(np.ascontiguousarray(a)) for a in (q[:, :L], k[:, :L], q[:, L:], k[:, L:]))
    vt_t, vt_i = _dev(_vt(v[:, :L], Lp)), _dev(_vt(v[:, L:], Np))
    o = torch.empty((L + N, heads * 128), dtype=torch.int16, device="cuda")
    qi.block_causal_attention(heads, L, N, qi.QI_MODE_JOINT, q_t, k_t, vt_t, q_i, k_i, vt_i, o)
    got = bf16_vals(host(o).view(np.uint16)).reshape(L + N, heads, 128).transpose(1, 0, 2)
    o_t, o_i = dit.block_causal_attention(qv[:, :L], kv[:, :L], vv[:, :L], qv[:, L:], kv[:, L:], vv[:, L:])
    ref = np.concatenate([o_t, o_i], axis=1)
    assert np.all(np.isfinite(got))
    rel = dit.rel_l2(got, ref)
    mx = np.max(np.abs(got - ref))
    log(f"  rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert rel < 1e-2 and mx < 5e-2
    o2 = torch.empty((N, heads * 128), dtype=torch.int16, device="cuda")
    qi.block_causal_attention(heads, L, N, qi.QI_MODE_IMAGE_ONLY, None, k_t, vt_t, q_i, k_i, vt_i, o2)
    assert_bits_equal(host(o2), host(o)[L:], "image-only attention rows")


def test_attention_text_rows_ignore_image_keys():
    import torch
    heads, L, N = 2, 70, 90
    q, k, v = _attn_inputs(heads, L, N, seed=40)
    Lp, Np = 128, 128
    args = [_dev(np.ascontiguousarray(a)) for a in (q[:, :L], k[:, :L])]
    vt_t = _dev(_vt(v[:, :L], Lp))
    outs = []
    for s in (50, 60):
        q2, k2, v2 = _attn_inputs(heads, L, N, seed=s)
        o = torch.empty((L + N, heads * 128), dtype=torch.int16, device="cuda")
        qi.block_causal_attention(heads, L, N, qi.QI_MODE_JOINT, args[0], args[1], vt_t,
                                  _dev(np.ascontiguousarray(q2[:, L:])), _dev(np.ascontiguousarray(k2[:, L:])),
                                  _dev(_vt(v2[:, L:], Np)), o)
        outs.append(host(o))
    assert np.array_equal(outs[0][:L], outs[1][:L])
    assert not np.array_equal(outs[0][L:], outs[1][L:])


@pytest.mark.parametrize("wl_id,t", [(1, 0.7), (2, 0.7), (2, 0.0), (2, 1.0)])
def test_modulation_matches_oracle(wl_id, t):
    import torch
    wl = qs.workload(wl_id)
    sw = qs.shared_weights(wl, as_bf16=True)
    dims = qi.make_dims(wl.hidden, wl.ffn, 1, wl.txt_dim)
    mod = torch.empty((2, 4 * wl.hidden), dtype=torch.float32, device="cuda")
    qi.modulation(dims, _dev(sw["w_mod"]), _dev(sw["b_mod"]), t, mod)
    got = host(mod)
    m_txt, m_img = dit.modulation_rows(bf16_vals(sw["w_mod"]), sw["b_mod"], np.float32(t), wl.hidden)
    for g, r in ((got[0], m_txt), (got[1], m_img)):
        assert np.max(np.abs(g - r)) < 1e-5 * max(1.0, np.max(np.abs(r))) * 8


@pytest.mark.parametrize("n", [1, 3, 4, 64, 4096 * 64, 4096 * 64 + 3])
def test_euler_update_bit_exact(n):
    import torch
    x = qs.normal_array((n,), seed=5)
    v = qs.normal_array((n,), seed=6)
    s, _ = qi.flow_sigmas(40, 4096)
    xd = torch.from_numpy(x.copy()).cuda()
    qi.euler_update(xd, torch.from_numpy(v).cuda(), s[3], s[4])
    ref = dit.euler_update(x, v, s[3], s[4])
    assert_bits_equal(host(xd), ref, "euler")
