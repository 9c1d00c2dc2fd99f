"""ctypes view of libqi.so: the C structs of include/qi.h and the exported
symbols with their signatures.  Loading fails loudly when the library is not
built; there is no fallback path."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libqi.so")

QI_OK = 0
QI_ERR_NULL = -1
QI_ERR_SHAPE = -2
QI_ERR_RANGE = -3
QI_ERR_ALIGN = -4
QI_ERR_WORKSPACE = -5
QI_ERR_CACHE = -6
QI_ERR_HIP = -7
QI_ERR_UNSUPPORTED = -8
QI_MODE_JOINT = 0
QI_MODE_IMAGE_ONLY = 1
QI_NOALLOC_SCRATCH_BYTES = 160 * 1024 * 1024


class QiDims(Structure):
    _fields_ = [("hidden", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("n_blocks", c_int32), ("txt_dim", c_int32)]


class QiBlockW(Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("w_gu", c_void_p),
                ("w_down", c_void_p), ("norm1", c_void_p), ("norm2", c_void_p)]


class QiModelW(Structure):
    _fields_ = [("blocks", POINTER(QiBlockW)),
                ("w_mod", c_void_p), ("b_mod", c_void_p),
                ("w_img", c_void_p), ("b_img", c_void_p),
                ("txt_norm", c_void_p), ("w_txt", c_void_p), ("b_txt", c_void_p),
                ("norm_out", c_void_p), ("w_out", c_void_p), ("b_out", c_void_p)]


class QiKvCache(Structure):
    _fields_ = [("kv", c_void_p), ("L", c_int32), ("n_blocks", c_int32),
                ("hidden", c_int32), ("valid", c_int32)]


class QiEncDims(Structure):
    _fields_ = [("hidden", c_int32), ("heads", c_int32), ("kv_heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("n_layers", c_int32), ("vocab", c_int32)]


class QiEncLayerW(Structure):
    _fields_ = [("w_qkv", c_void_p), ("q_norm", c_void_p), ("k_norm", c_void_p), ("w_o", c_void_p),
                ("w_gu", c_void_p), ("w_down", c_void_p), ("in_norm", c_void_p), ("post_norm", c_void_p)]


class QiEncModelW(Structure):
    _fields_ = [("layers", POINTER(QiEncLayerW)), ("embed", c_void_p)]


_P = POINTER
# name -> (restype, argtypes); every symbol include/qi.h declares
SIGNATURES = {
    "qi_status_str": (c_char_p, [c_int32]),
    "qi_version": (c_char_p, []),
    "qi_rope_axis_table": (c_int32, [c_int32, c_void_p, c_void_p]),
    "qi_rope_tables": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "qi_flow_sigmas": (c_int32, [c_int32, c_int32, c_void_p, c_void_p]),
    "qi_workspace_bytes": (c_size_t, [_P(QiDims), c_int32, c_int32]),
    "qi_kv_slot_elems": (c_size_t, [_P(QiDims), c_int32]),
    "qi_kv_cache_bytes": (c_size_t, [_P(QiDims), c_int32]),
    "qi_dit_block_fwd": (c_int32, [_P(QiDims), _P(QiBlockW), c_int32, c_int32, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qi_dit_step": (c_int32, [_P(QiDims), _P(QiModelW), c_int32, c_int32, c_void_p, c_void_p, c_float,
                              c_void_p, c_void_p, c_void_p, c_void_p, _P(QiKvCache), c_void_p,
                              c_void_p, c_size_t, c_void_p]),
    "qi_dit_step_noalloc": (c_int32, [_P(QiDims), _P(QiModelW), c_int32, c_int32, c_void_p, c_void_p, c_float,
                                      c_void_p, c_void_p, c_void_p, c_void_p, _P(QiKvCache), c_void_p, c_void_p]),
    "qi_text_kv_capture": (c_int32, [_P(QiDims), _P(QiModelW), c_int32, c_int32, c_void_p, c_void_p,
                                     c_float, c_void_p, c_void_p, c_void_p, c_void_p, _P(QiKvCache),
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "qi_euler_update": (c_int32, [c_void_p, c_void_p, c_float, c_float, c_int64, c_void_p]),
    "qi_cfg_workspace_bytes": (c_size_t, [_P(QiDims), c_int32]),
    "qi_dit_step_cfg": (c_int32, [_P(QiDims), _P(QiModelW), c_int32, c_void_p, c_float, c_void_p, c_void_p,
                                  _P(QiKvCache), _P(QiKvCache), c_void_p, c_void_p, c_size_t, c_void_p]),
    "qi_euler_update_cfg": (c_int32, [c_void_p, c_void_p, c_float, c_float, c_float, c_int64, c_void_p]),
    "qi_fbc_bytes": (c_size_t, [_P(QiDims), c_int32]),
    "qi_enc_rope_table": (c_int32, [c_int32, c_float, c_void_p, c_void_p]),
    "qi_enc_workspace_bytes": (c_size_t, [_P(QiEncDims), c_int32]),
    "qi_text_encoder_fwd": (c_int32, [_P(QiEncDims), _P(QiEncModelW), c_void_p, c_int32, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_size_t, c_void_p]),
    "qi_dpmpp_2m_coeffs": (c_int32, [c_int32, c_float, c_float, c_float, c_void_p]),
    "qi_dpmpp_2m_update": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_float, c_float, c_float, c_int64,
                                     c_void_p]),
    "qi_fbc_reset": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "qi_dit_step_fbc": (c_int32, [_P(QiDims), _P(QiModelW), c_int32, c_int32, c_void_p, c_float, c_void_p,
                                  c_void_p, _P(QiKvCache), c_float, c_void_p, c_size_t, c_void_p, c_void_p,
                                  c_size_t, c_void_p]),
    "qi_fbc_stats": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "qi_modulation": (c_int32, [_P(QiDims), c_void_p, c_void_p, c_float, c_void_p, c_void_p]),
    "qi_block_causal_attention": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "qi_linear_bf16": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p]),
    "qi_kernel_kind_name": (c_char_p, [c_int32]),
    "qi_timing_begin": (c_int32, [c_int32]),
    "qi_timing_end": (c_int32, [c_void_p, c_void_p, c_void_p]),
}
# the bench-only calibration library (include/qi_calib.h, lib/libqi_calib.so)
CALIB_PATH = os.path.join(PKG, "lib", "libqi_calib.so")
CALIB_SIGNATURES = {
    "qi_calib_mfma_tflops": (c_int32, [c_int32, c_int32, c_void_p]),
    "qi_calib_copy_gbs": (c_int32, [c_void_p, c_void_p, c_int64, c_int32, c_void_p]),
    "qi_calib_read_gbs": (c_int32, [c_void_p, c_int64, c_void_p, c_int32, c_void_p]),
    "qi_calib_lds_cycles": (c_int32, [c_int32, c_int32, c_void_p]),
    "qi_calib_valu_ns": (c_int32, [c_int32, c_int32, c_void_p]),
}
QI_KERNEL_KINDS = 16

_lib = None
_calib = None


class QiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: qi status {status} ({status_str(status)})")


def load(path: str | None = None):
    """Load libqi.so (once).  Raises if it is missing: the HIP library is the
    only implementation of the step."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library {p} is not built; run "
                           "`python -m block_causal_attention_qi_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def load_calib():
    """Load the bench-only calibration library libqi_calib.so (once)."""
    global _calib
    if _calib is not None:
        return _calib
    if not os.path.exists(CALIB_PATH):
        raise RuntimeError(f"calibration library {CALIB_PATH} is not built; run "
                           "`python -m block_causal_attention_qi_amd.build`")
    lib = ctypes.CDLL(CALIB_PATH)
    for name, (res, args) in CALIB_SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _calib = lib
    return lib


def status_str(s: int) -> str:
    try:
        return load().qi_status_str(int(s)).decode()
    except Exception:  # pragma: no cover
        return "?"


def check(status: int, where: str):
    if status != QI_OK:
        raise QiError(status, where)
