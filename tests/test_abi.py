"""The C ABI on the CPU: the library loads, exports every symbol include/qi.h
declares, computes the host tables exactly like the oracle, and rejects bad
arguments on the host before anything is enqueued.  No GPU compute is called:
the argument-rejection tests pass fake device addresses that the validation
must refuse, and they are skipped where a GPU is visible so a validation bug
can never launch a kernel on them."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_causal_attention_qi_amd as qi
from block_causal_attention_qi_amd import _lib
from oracle import dit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols(header="qi.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qi_[a-z0-9_]+)\s*\(", src)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer validation tests run only without a GPU")


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load()
    decl = _declared_symbols("qi.h")
    assert len(decl) >= 20 and "qi_dit_step" in decl
    for name in decl:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding misses {name}"
    assert lib.qi_version().decode().startswith("qi-dit-gfx950")
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["qi.h", "qi_calib.h"], headers


def test_calibration_library_is_separate():
    """The calibration microbenchmarks (which allocate, create a stream and
    block) live in their own bench-only library, not in libqi."""
    lib = _lib.load()
    cal = _lib.load_calib()
    decl = _declared_symbols("qi_calib.h")
    assert len(decl) == 5
    for name in decl:
        assert hasattr(cal, name), name
        assert name in _lib.CALIB_SIGNATURES, f"binding misses {name}"
    import subprocess
    syms = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "qi_dit_step" in syms and "qi_calib" not in syms


def test_status_strings():
    for s in range(-8, 1):
        assert len(_lib.status_str(s)) >= 2 and _lib.status_str(s) != "unknown status"


@pytest.mark.parametrize("d", [16, 56])
def test_axis_table_bit_exact_with_oracle(d):
    c, s = qi.rope_axis_table(d)
    oc, os_ = dit.rope_axis_table(d)
    assert c.tobytes() == oc.tobytes() and s.tobytes() == os_.tobytes()


@pytest.mark.parametrize("L,h,w", [(8, 8, 8), (22, 16, 16), (407, 64, 64), (494, 24, 24), (512, 128, 128), (9, 5, 3)])
def test_rope_rows_bit_exact_with_oracle(L, h, w):
    got = qi.rope_tables(L, h, w)
    ref = dit.rope_rows(L, h, w)
    for g, r in zip(got, ref):
        assert g.shape == r.shape and g.tobytes() == r.tobytes()


@pytest.mark.parametrize("steps,n", [(40, 256), (40, 1024), (40, 4096), (40, 576), (40, 16384), (25, 4096), (2, 64)])
def test_flow_sigmas_bit_exact_with_oracle(steps, n):
    s, t = qi.flow_sigmas(steps, n)
    os_, ot = dit.flow_sigmas(steps, n)
    assert s.tobytes() == os_.tobytes() and t.tobytes() == ot.tobytes()


def test_host_table_errors():
    lib = _lib.load()
    buf = np.zeros(9216 * 64, np.float32)
    p = buf.ctypes.data
    assert lib.qi_rope_axis_table(15, p, p) == _lib.QI_ERR_RANGE
    assert lib.qi_rope_axis_table(16, None, p) == _lib.QI_ERR_NULL
    assert lib.qi_rope_tables(8, 0, 8, p, p, p, p) == _lib.QI_ERR_RANGE
    assert lib.qi_rope_tables(8, 4096, 8, p, p, p, p) == _lib.QI_ERR_RANGE   # rows below -1024
    assert lib.qi_rope_tables(8, 8, 8, None, p, p, p) == _lib.QI_ERR_NULL
    assert lib.qi_flow_sigmas(1, 256, p, p) == _lib.QI_ERR_RANGE
    assert lib.qi_flow_sigmas(40, 0, p, p) == _lib.QI_ERR_RANGE
    assert lib.qi_flow_sigmas(40, 256, None, p) == _lib.QI_ERR_NULL


def _dims(**over):
    d = dict(hidden=4096, heads=32, head_dim=128, ffn=12288, n_blocks=32, txt_dim=4096)
    d.update(over)
    return _lib.QiDims(**d)


def test_sizes():
    d = _dims()
    assert qi.workspace_bytes(d, 407, 4096) > 0
    # cache: 2 x blocks x L x H bf16 plus the V^T padding of L to 64
    L = 494
    assert qi.kv_cache_bytes(d, L) == 32 * 32 * 128 * (L + 512) * 2
    assert qi.workspace_bytes(_dims(head_dim=64), 8, 64) == 0
    assert qi.workspace_bytes(_dims(heads=31), 8, 64) == 0
    assert qi.workspace_bytes(d, 0, 64) == 0 and qi.workspace_bytes(d, 513, 64) == 0
    assert qi.workspace_bytes(d, 8, 16385) == 0


FAKE = 1 << 40          # 16-byte aligned, never dereferenced: validation must refuse first
FAKE_MIS = FAKE + 4


def _fake_model(n_blocks=1, mis=None):
    bw = (_lib.QiBlockW * n_blocks)()
    for i in range(n_blocks):
        bw[i] = _lib.QiBlockW(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    vals = [FAKE] * 10
    if mis is not None:
        vals[mis] = FAKE_MIS
    return bw, _lib.QiModelW(ctypes.cast(bw, ctypes.POINTER(_lib.QiBlockW)), *vals)


@no_gpu_only
def test_step_rejects_bad_arguments_on_the_host():
    lib = _lib.load()
    d = _dims(n_blocks=1)
    bw, mw = _fake_model(1)
    ws = qi.workspace_bytes(d, 22, 256)
    good = dict(L=22, N=256, img=FAKE, txt=FAKE, t=0.5, tc=FAKE, ts=FAKE, ic=FAKE, is_=FAKE,
                cache=None, vel=FAKE, ws=FAKE, wsb=ws)

    def call(dims=d, model=mw, **over):
        a = dict(good)
        a.update(over)
        return lib.qi_dit_step(ctypes.byref(dims), ctypes.byref(model), a["L"], a["N"], a["img"], a["txt"],
                               a["t"], a["tc"], a["ts"], a["ic"], a["is_"], a["cache"], a["vel"], a["ws"],
                               a["wsb"], None)

    assert call(wsb=ws - 1) == _lib.QI_ERR_WORKSPACE
    assert call(L=0) == _lib.QI_ERR_RANGE
    assert call(L=513) == _lib.QI_ERR_RANGE
    assert call(N=0, wsb=ws) == _lib.QI_ERR_RANGE
    assert call(N=16385) == _lib.QI_ERR_RANGE
    assert call(t=1.5, wsb=ws - 1) == _lib.QI_ERR_RANGE
    assert call(t=float("nan"), wsb=ws - 1) == _lib.QI_ERR_RANGE
    assert call(img=None, wsb=ws - 1) == _lib.QI_ERR_NULL
    assert call(txt=None, wsb=ws - 1) == _lib.QI_ERR_NULL        # joint pass needs txt_feats
    assert call(img=FAKE_MIS, wsb=ws - 1) == _lib.QI_ERR_ALIGN
    assert call(dims=_dims(n_blocks=1, hidden=4000), wsb=ws - 1) == _lib.QI_ERR_SHAPE
    _, bad_model = _fake_model(1, mis=0)
    assert call(model=bad_model, wsb=ws - 1) == _lib.QI_ERR_ALIGN
    bw_null = (_lib.QiBlockW * 1)()
    bw_null[0] = _lib.QiBlockW(FAKE, 0, FAKE, FAKE, FAKE, FAKE)
    mw_null = _lib.QiModelW(ctypes.cast(bw_null, ctypes.POINTER(_lib.QiBlockW)), *([FAKE] * 10))
    assert call(model=mw_null, wsb=ws - 1) == _lib.QI_ERR_NULL

    # a stale or mismatched cache is refused with QI_ERR_CACHE (full workspace,
    # so nothing else is wrong)
    stale = _lib.QiKvCache(FAKE, 22, 1, 4096, 0)
    assert call(cache=ctypes.byref(stale)) == _lib.QI_ERR_CACHE
    other_L = _lib.QiKvCache(FAKE, 21, 1, 4096, 1)
    assert call(cache=ctypes.byref(other_L)) == _lib.QI_ERR_CACHE
    other_blocks = _lib.QiKvCache(FAKE, 22, 2, 4096, 1)
    assert call(cache=ctypes.byref(other_blocks)) == _lib.QI_ERR_CACHE
    other_h = _lib.QiKvCache(FAKE, 22, 1, 2048, 1)
    assert call(cache=ctypes.byref(other_h)) == _lib.QI_ERR_CACHE
    assert call(vel=None) == _lib.QI_ERR_NULL


@no_gpu_only
def test_capture_block_and_component_reject_bad_arguments():
    lib = _lib.load()
    d = _dims(n_blocks=1)
    bw, mw = _fake_model(1)
    ws = qi.workspace_bytes(d, 22, 256)
    cache = _lib.QiKvCache(0, 0, 0, 0, 0)
    assert lib.qi_text_kv_capture(ctypes.byref(d), ctypes.byref(mw), 22, 256, FAKE, FAKE, 0.5, FAKE, FAKE,
                                  FAKE, FAKE, ctypes.byref(cache), FAKE, FAKE, ws, None) == _lib.QI_ERR_NULL
    assert lib.qi_text_kv_capture(ctypes.byref(d), ctypes.byref(mw), 22, 256, FAKE, FAKE, 0.5, FAKE, FAKE,
                                  FAKE, FAKE, None, FAKE, FAKE, ws, None) == _lib.QI_ERR_NULL
    blk = _lib.QiBlockW(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    f = lib.qi_dit_block_fwd
    assert f(ctypes.byref(d), ctypes.byref(blk), 22, 256, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws,
             None) == _lib.QI_ERR_CACHE   # image-only pass without text K/V
    assert f(ctypes.byref(d), ctypes.byref(blk), 22, 256, 2, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws,
             None) == _lib.QI_ERR_RANGE
    assert f(ctypes.byref(d), ctypes.byref(blk), 22, 256, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 256,
             None) == _lib.QI_ERR_WORKSPACE
    assert f(ctypes.byref(d), ctypes.byref(blk), 22, 256, 0, FAKE_MIS, FAKE, FAKE, FAKE, None, FAKE, ws,
             None) == _lib.QI_ERR_ALIGN
    assert lib.qi_euler_update(FAKE, FAKE, 1.0, 0.9, -1, None) == _lib.QI_ERR_RANGE
    assert lib.qi_euler_update(FAKE, FAKE, 1.0, 0.9, 0, None) == _lib.QI_OK      # no-op
    assert lib.qi_euler_update(None, FAKE, 1.0, 0.9, 5, None) == _lib.QI_ERR_NULL
    assert lib.qi_euler_update(FAKE_MIS, FAKE, 1.0, 0.9, 5, None) == _lib.QI_ERR_ALIGN
    a = lib.qi_block_causal_attention
    assert a(32, 0, 256, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.QI_ERR_RANGE
    assert a(32, 22, 256, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.QI_ERR_NULL
    assert a(32, 22, 256, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE_MIS, None) == _lib.QI_ERR_ALIGN
    g = lib.qi_linear_bf16
    assert g(64, 100, 64, FAKE, FAKE, None, FAKE, None) == _lib.QI_ERR_RANGE
    assert g(64, 128, 96, FAKE, FAKE, None, FAKE, None) == _lib.QI_ERR_RANGE
    assert g(64, 128, 64, None, FAKE, None, FAKE, None) == _lib.QI_ERR_NULL
    cal = _lib.load_calib()
    c = cal.qi_calib_mfma_tflops
    out = ctypes.c_double(0)
    assert c(2, 10, ctypes.byref(out)) == _lib.QI_ERR_RANGE
    assert c(0, 10, None) == _lib.QI_ERR_NULL
    assert cal.qi_calib_copy_gbs(FAKE, FAKE, 15, 1, ctypes.byref(out)) == _lib.QI_ERR_RANGE
    assert cal.qi_calib_copy_gbs(FAKE_MIS, FAKE, 64, 1, ctypes.byref(out)) == _lib.QI_ERR_ALIGN
    assert cal.qi_calib_read_gbs(FAKE, 15, FAKE, 1, ctypes.byref(out)) == _lib.QI_ERR_RANGE
    assert cal.qi_calib_read_gbs(FAKE_MIS, 64, FAKE, 1, ctypes.byref(out)) == _lib.QI_ERR_ALIGN
    assert cal.qi_calib_read_gbs(FAKE, 64, None, 1, ctypes.byref(out)) == _lib.QI_ERR_NULL
    assert cal.qi_calib_lds_cycles(5, 100, ctypes.byref(out)) == _lib.QI_ERR_RANGE
    assert cal.qi_calib_lds_cycles(0, 3, ctypes.byref(out)) == _lib.QI_ERR_RANGE
    assert cal.qi_calib_lds_cycles(0, 100, None) == _lib.QI_ERR_NULL
    m = lib.qi_modulation
    assert m(ctypes.byref(d), FAKE, FAKE, 2.0, FAKE, None) == _lib.QI_ERR_RANGE
    assert m(ctypes.byref(d), None, FAKE, 0.5, FAKE, None) == _lib.QI_ERR_NULL
