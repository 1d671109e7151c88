"""ctypes binding of the C ABI declared in ``include/xcorr.h``.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libxcorr_hip.so``.  Loading fails loudly when the library has not
been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libxcorr_hip.so")

# Status codes (include/xcorr.h)
XC_OK = 0
XC_ERR_NULL = -1
XC_ERR_SHAPE = -2
XC_ERR_TEMPLATE_WIDTH = -3
XC_ERR_OVERFLOW = -4
XC_ERR_ALIGN = -5
XC_ERR_HIP = -6
XC_ERR_VARIANT = -7
XC_ERR_SCRATCH = -8

XC_NCC_AUTO = 0
XC_NCC_DOT4_ILP = 1
XC_NCC_DOT4_C1 = 2
XC_NCC_SCALAR_C1 = 3
XC_NCC_MFMA = 4
XC_NCC_DOT4_ILP_Q1 = 5
XC_NCC_DOT4_ILP_Q2 = 6
XC_NCC_DOT4_ILP_Q4 = 7
XC_NCC_MFMA_W4 = 8
XC_NCC_MFMA_W2 = 9
XC_NCC_DOT4_COLS1 = 10
XC_NCC_DOT4_COLS2 = 11
XC_NCC_DOT4_COLS4 = 12
XC_NCC_DOT4_COLS8 = 13
XC_NCC_MFMA32 = 14

XC_NCC_MODE_VALID = 0
XC_NCC_MODE_SAME = 1
XC_NCC_MODE_FULL = 2

XC_XCORR_AUTO = 0
XC_XCORR_OVERLAP = 1
XC_XCORR_BLOCKDIAG = 2
XC_XCORR_WAVE = 3
XC_XCORR_SMALL = 4
XC_XCORR_MFMA = 5

XC_NCC_MAX_TEMPLATE_PIXELS = 66051

# Every symbol the public header declares.
EXPORTED = ("ncc_u8_run", "ncc_u8_run_variant", "ncc_u8_peak", "ncc_u8_auto_variant", "ncc_u8_mode_workspace",
            "ncc_u8_run_mode", "ncc_u8_run_mode_noalloc",
            "xcorr_f32_run", "xcorr_f32_run_algo", "xc_status_str")

# xc_ncc_peak (include/xcorr.h): key u64, y i32, x i32, coef f32, reserved i32
PEAK_BYTES = 24


class XcError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int


def load(path: str = LIB_PATH):
    """Load ``libxcorr_hip.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.ncc_u8_run.restype = _i
    lib.ncc_u8_run.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp]
    lib.ncc_u8_run_variant.restype = _i
    lib.ncc_u8_run_variant.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _i, _vp]
    lib.ncc_u8_peak.restype = _i
    lib.ncc_u8_peak.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp]
    lib.ncc_u8_auto_variant.restype = _i
    lib.ncc_u8_auto_variant.argtypes = [_i, _i, _i, _i, ctypes.POINTER(ctypes.c_int)]
    lib.ncc_u8_mode_workspace.restype = _i
    lib.ncc_u8_mode_workspace.argtypes = [_i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_size_t)]
    lib.ncc_u8_run_mode.restype = _i
    lib.ncc_u8_run_mode.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _i, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp, _i,
                                    _vp]
    lib.ncc_u8_run_mode_noalloc.restype = _i
    lib.ncc_u8_run_mode_noalloc.argtypes = [_vp, _i, _i, _i, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i, _vp]
    lib.xcorr_f32_run.restype = _i
    lib.xcorr_f32_run.argtypes = [_vp, _i, _vp, _i, _i, _i, _vp, _vp]
    lib.xcorr_f32_run_algo.restype = _i
    lib.xcorr_f32_run_algo.argtypes = [_vp, _i, _vp, _i, _i, _i, _vp, _i, _vp]
    lib.xc_status_str.restype = ctypes.c_char_p
    lib.xc_status_str.argtypes = [_i]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().xc_status_str(status).decode()


def check(status: int, where: str) -> None:
    if status != XC_OK:
        raise XcError(status, where)


def ncc_u8_run(image, width, height, pitch, tmpl, t_width, t_height, sum_i, sum_isq, sum_it, coef,
               stream=None, variant=XC_NCC_AUTO) -> int:
    """Raw call with integer device addresses (0 for NULL); returns the status."""
    return load().ncc_u8_run_variant(image, width, height, pitch, tmpl, t_width, t_height,
                                     sum_i or None, sum_isq or None, sum_it or None, coef or None,
                                     variant, stream or None)


def ncc_u8_peak(image, width, height, pitch, tmpl, t_width, t_height, sum_i, sum_isq, sum_it, coef, peak,
                stream=None, variant=XC_NCC_AUTO) -> int:
    """Raw call with integer device addresses (0 for NULL; ``peak`` points to
    PEAK_BYTES of device memory); returns the status."""
    return load().ncc_u8_peak(image, width, height, pitch, tmpl, t_width, t_height,
                              sum_i or None, sum_isq or None, sum_it or None, coef or None, peak or None,
                              variant, stream or None)


def ncc_u8_auto_variant(width, height, t_width, t_height) -> tuple[int, int]:
    """(status, variant) that ncc_u8_run picks for these shapes (host-only)."""
    v = ctypes.c_int(-1)
    st = load().ncc_u8_auto_variant(width, height, t_width, t_height, ctypes.byref(v))
    return st, v.value


def ncc_u8_mode_workspace(width, height, t_width, t_height, mode) -> tuple[int, int]:
    """(status, workspace bytes) for an output mode."""
    n = ctypes.c_size_t(0)
    st = load().ncc_u8_mode_workspace(width, height, t_width, t_height, mode, ctypes.byref(n))
    return st, n.value


def ncc_mode_shape(width, height, t_width, t_height, mode) -> tuple[int, int]:
    """(out_h, out_w) of an output mode (include/xcorr.h, ncc_u8_run_mode)."""
    if mode == XC_NCC_MODE_SAME:
        return height, width
    if mode == XC_NCC_MODE_FULL:
        return height + t_height - 1, width + t_width - 1
    return height - t_height + 1, width - t_width + 1


def ncc_u8_run_mode(image, width, height, pitch, tmpl, t_width, t_height, mode, workspace, workspace_bytes,
                    sum_i, sum_isq, sum_it, coef, stream=None, variant=XC_NCC_AUTO) -> int:
    """Raw call with integer device addresses (0 for NULL); returns the status."""
    return load().ncc_u8_run_mode(image, width, height, pitch, tmpl, t_width, t_height, mode, workspace or None,
                                  workspace_bytes, sum_i or None, sum_isq or None, sum_it or None, coef or None,
                                  variant, stream or None)


XC_NCC_MODE_SCRATCH_BYTES = 16 << 20


def ncc_u8_run_mode_noalloc(image, width, height, pitch, tmpl, t_width, t_height, mode, sum_i, sum_isq, sum_it,
                            coef, stream=None, variant=XC_NCC_AUTO) -> int:
    """Raw call with integer device addresses (0 for NULL); returns the status."""
    return load().ncc_u8_run_mode_noalloc(image, width, height, pitch, tmpl, t_width, t_height, mode,
                                          sum_i or None, sum_isq or None, sum_it or None, coef or None, variant,
                                          stream or None)


def decode_peak(raw: bytes) -> tuple[int, int, float]:
    """(y, x, coef) from the PEAK_BYTES of an xc_ncc_peak read back to the host."""
    import struct
    _key, y, x, coef, _res = struct.unpack("<QiifI", bytes(raw[:PEAK_BYTES]))
    return y, x, coef


def xcorr_f32_run(left, n_left, right, n_right, rows, cols, out, stream=None, algo=XC_XCORR_AUTO) -> int:
    """Raw call with integer device addresses; returns the status."""
    return load().xcorr_f32_run_algo(left, n_left, right, n_right, rows, cols, out, algo, stream or None)
