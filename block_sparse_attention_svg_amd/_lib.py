"""ctypes declarations of libsvg.so (include/svg.h).  Loading fails loudly when
the library has not been built; there is no fallback implementation."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvg.so")

SVG_OK = 0
SVG_ERR_INVALID_ARG = 1
SVG_ERR_UNSUPPORTED = 2
SVG_ERR_CAPACITY = 3
SVG_ERR_HIP = 4
SVG_BF16 = 0
SVG_F32 = 1


class SvgShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "H", "N", "D", "F", "Hs", "Ws", "block")]


class SvgMask(ctypes.Structure):
    _fields_ = [
        ("n_masks", ctypes.c_int), ("n_qb", ctypes.c_int), ("n_kb", ctypes.c_int),
        ("bitmap", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p), ("iv", ctypes.c_void_p),
    ]


class SvgRope(ctypes.Structure):
    _fields_ = [("d_f", ctypes.c_int), ("d_y", ctypes.c_int), ("d_x", ctypes.c_int),
                ("theta", ctypes.c_float)]


class SvgError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "svg_build_masks": (_I, [SvgShape, _I, _P, _P]),
    "svg_encode_iv_capacity": (ctypes.c_int64, [_I, _I, _I]),
    "svg_encode_mask": (_I, [_P, _I, _I, _I, _P, _P, _P, ctypes.c_int64, _P]),
    "svg_permute": (_I, [_P, _P, _I, SvgShape, _P, _I, _P]),
    "svg_qk_norm_rope": (_I, [_P, _P, SvgShape, _I, _P, ctypes.c_float, ctypes.POINTER(SvgRope), _P, _P]),
    "svg_profile_workspace_bytes": (ctypes.c_size_t, [SvgShape, _I]),
    "svg_profile_heads": (_I, [_P, _P, _P, SvgShape, ctypes.c_float, _P, _I,
                               ctypes.POINTER(SvgMask), _P, _P, _P, ctypes.c_size_t, _P]),
    "svg_block_sparse_attn": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, SvgShape, ctypes.c_float,
                                   ctypes.POINTER(SvgMask), _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "svg_attn_workspace_bytes": (ctypes.c_size_t, [SvgShape, _I]),
    "svg_vt_bytes": (ctypes.c_size_t, [SvgShape]),
    "svg_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "svg_fp8_vt_bytes": (ctypes.c_size_t, [SvgShape]),
    "svg_quantize_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, SvgShape, _P, _P]),
    "svg_block_sparse_attn_fp8": (_I, [_P, _P, _P, _P, _P, SvgShape, ctypes.c_float, ctypes.POINTER(SvgMask),
                                       _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "svg_block_sparse_attn_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, SvgShape, ctypes.c_float,
                                           ctypes.POINTER(SvgMask), _P, _P, _P, _P]),
    "svg_prepare_kv": (_I, [_P, _P, _P, _P, SvgShape, _P, _P]),
    "svg_row_broadcast": (_I, [_P, SvgShape, _P, _I, _P]),
    "svg_restrict_anchor_rows": (_I, [_P, _I, SvgShape, _P, _I, _P]),
    "svg_calibrate_masks": (_I, [_P, _I, _I, _I, ctypes.c_double, _P, _P]),
    "svg_block_energy": (_I, [_P, _P, SvgShape, ctypes.c_float, _P, _P]),
    "svg_aggregate_masks": (_I, [_P, _I, ctypes.c_int64, ctypes.c_double, _P, _P]),
    "svg_eps_schedule": (_I, [_I, _I, ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
    "svg_row_similarity_workspace_bytes": (ctypes.c_size_t, [SvgShape]),
    "svg_row_similarity": (_I, [_P, _P, SvgShape, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]),
    "svg_mfma_peak_probe": (_I, [_I, _I, _P, ctypes.c_int64, ctypes.POINTER(ctypes.c_double), _P]),
    "svg_status_string": (ctypes.c_char_p, [_I]),
    "svg_last_error": (ctypes.c_char_p, []),
    "svg_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library (raises if libsvg.so is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m block_sparse_attention_svg_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != SVG_OK:
        msg = lib().svg_last_error().decode(errors="replace")
        raise SvgError(fn, status, msg)
