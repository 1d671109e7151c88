"""CPU oracle for direct sliding-window correlation (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  Nothing in the GPU
library imports, links or calls this package, and this package imports
nothing from the GPU library.

Functions follow the definitions cited in ``oracle.c``:

* :func:`ncc_u8` -- u8 normalized correlation, "The CUDA Handbook" section
  15.5 "Instruction-Level Parallelism and DP4A" (the SumI / SumISq / SumIT
  accumulators over unsigned 8-bit pixels), coefficient read as Pearson's r.
* :func:`ncc_u8_mode` -- the same correlation over other output domains: the
  pages define the windows inside the image only; "same" and "full" read
  pixels outside the image as 0 (counted among the window's pixels), the
  zero-padding convention of scipy.signal.correlate2d, i.e. the valid-mode
  definition applied to the image with zero borders.
* :func:`ncc_peak` -- the best match of a coefficient map (first entry, in
  row-major order, holding the maximum), the usual last step of template
  matching.
* :func:`xcorr_f32` -- full 2D cross-correlation over all overlaps, JPDC 2023
  artifact README (each thread computes one overlap; one-to-one, one-to-many
  and multi-matrix-both groupings), accumulated in fp64.

Every function here has pins in ``tests/test_oracle_*.py`` that tie it to
closed forms, invariants and library routines rather than to itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)

ORACLE_OK = 0
ORACLE_ERR_ARG = -1
ORACLE_ERR_U32 = -2


def build(force: bool = True, extra_flags: tuple[str, ...] = (), src: str = _SRC, out: str = _LIB) -> str:
    """Compile ``oracle.c`` with gcc (plain -O2, OpenMP over independent outputs).

    ``src``/``out`` let the mutation tests build a deliberately broken copy
    into a temporary directory; the default builds the real oracle in place.
    """
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path: str):
    """Load a build of ``oracle.c`` and declare its C signatures.

    Every wrapper below takes ``lib=`` to run against such a handle instead
    of the default build (used by the mutation tests).
    """
    lib = ctypes.CDLL(path)
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_ncc_u8_rows.restype = ctypes.c_int
    lib.oracle_ncc_u8_rows.argtypes = [
        _u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, _u32p, _u32p, _u32p, _f32p, _f64p, ctypes.c_int]
    lib.oracle_ncc_u8_points.restype = ctypes.c_int
    lib.oracle_ncc_u8_points.argtypes = [
        _u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p, ctypes.c_int, ctypes.c_int,
        _i32p, _i32p, ctypes.c_int64, _u32p, _u32p, _u32p, _f32p, _f64p, ctypes.c_int]
    lib.oracle_ncc_peak.restype = ctypes.c_int
    lib.oracle_ncc_peak.argtypes = [_f32p, ctypes.c_int64, _i64p, _f32p]
    lib.oracle_xcorr_f32.restype = ctypes.c_int
    lib.oracle_xcorr_f32.argtypes = [
        _f32p, ctypes.c_int, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    lib.oracle_xcorr_f32_points.restype = ctypes.c_int
    lib.oracle_xcorr_f32_points.argtypes = [
        _f32p, ctypes.c_int, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64p, ctypes.c_int64,
        _f64p, _f64p, ctypes.c_int]
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def _ptr(a: np.ndarray | None, ct):
    if a is None:
        return ctypes.cast(None, ct)
    return a.ctypes.data_as(ct)


def max_threads(lib=None) -> int:
    return int((lib or _load()).oracle_max_threads())


def _image_args(image: np.ndarray, width: int, height: int, tmpl: np.ndarray):
    image = np.ascontiguousarray(image, dtype=np.uint8)
    tmpl = np.ascontiguousarray(tmpl, dtype=np.uint8)
    if image.ndim != 2 or image.shape[0] != height or image.shape[1] < width:
        raise ValueError("image must be (height, pitch) with pitch >= width")
    if tmpl.ndim != 2:
        raise ValueError("template must be 2D")
    return image, tmpl


def ncc_u8(image: np.ndarray, width: int, height: int, tmpl: np.ndarray, *,
           y_begin: int = 0, y_end: int | None = None, nthreads: int = 0, lib=None) -> dict:
    """Valid-mode u8 normalized correlation for output rows [y_begin, y_end).

    ``image`` is (height, pitch) uint8 with pitch >= width; ``tmpl`` is dense
    (t_height, t_width).  Returns a dict of arrays ``sum_i``, ``sum_isq``,
    ``sum_it`` (uint32), ``coef`` (float32) and ``coef64`` (the fp64 value
    before rounding), each (rows, width - t_width + 1).
    Raises ``OverflowError`` when a window sum does not fit in 32 bits.
    """
    image, tmpl = _image_args(image, width, height, tmpl)
    th, tw = tmpl.shape
    out_h, out_w = height - th + 1, width - tw + 1
    if y_end is None:
        y_end = out_h
    rows = y_end - y_begin
    res = {k: np.empty((rows, out_w), dtype=np.uint32) for k in ("sum_i", "sum_isq", "sum_it")}
    res["coef"] = np.empty((rows, out_w), dtype=np.float32)
    res["coef64"] = np.empty((rows, out_w), dtype=np.float64)
    st = (lib or _load()).oracle_ncc_u8_rows(
        _ptr(image, _u8p), width, height, image.shape[1], _ptr(tmpl, _u8p), tw, th, y_begin, y_end,
        _ptr(res["sum_i"], _u32p), _ptr(res["sum_isq"], _u32p), _ptr(res["sum_it"], _u32p),
        _ptr(res["coef"], _f32p), _ptr(res["coef64"], _f64p), nthreads)
    if st == ORACLE_ERR_U32:
        raise OverflowError("a window sum does not fit in 32 bits")
    if st != ORACLE_OK:
        raise ValueError(f"oracle_ncc_u8_rows: bad arguments (status {st})")
    return res


MODE_VALID, MODE_SAME, MODE_FULL = 0, 1, 2


def ncc_mode_geometry(width: int, height: int, t_width: int, t_height: int, mode: int):
    """(out_h, out_w, pad_top, pad_left) of an output mode: output (y, x) is
    the window whose top-left pixel is (y - pad_top, x - pad_left)."""
    if mode == MODE_VALID:
        return height - t_height + 1, width - t_width + 1, 0, 0
    if mode == MODE_SAME:
        return height, width, (t_height - 1) // 2, (t_width - 1) // 2
    if mode == MODE_FULL:
        return height + t_height - 1, width + t_width - 1, t_height - 1, t_width - 1
    raise ValueError(f"unknown mode {mode}")


def ncc_u8_mode(image: np.ndarray, width: int, height: int, tmpl: np.ndarray, mode: int, *,
                nthreads: int = 0, lib=None) -> dict:
    """u8 normalized correlation in an output mode, written out as its
    definition: the image placed at (pad_top, pad_left) of a zero image large
    enough for every window of the mode, then the valid-mode oracle on it
    (so outside pixels are 0 and count among the window's pixels)."""
    image, tmpl = _image_args(image, width, height, tmpl)
    th, tw = tmpl.shape
    if mode == MODE_VALID:
        return ncc_u8(image, width, height, tmpl, nthreads=nthreads, lib=lib)
    out_h, out_w, pt, pl = ncc_mode_geometry(width, height, tw, th, mode)
    padded = np.zeros((out_h + th - 1, out_w + tw - 1), dtype=np.uint8)
    padded[pt:pt + height, pl:pl + width] = image[:, :width]
    return ncc_u8(padded, padded.shape[1], padded.shape[0], tmpl, nthreads=nthreads, lib=lib)


def ncc_u8_points(image: np.ndarray, width: int, height: int, tmpl: np.ndarray,
                  ys, xs, *, nthreads: int = 0, lib=None) -> dict:
    """The same quantities for selected windows (ys[k], xs[k]) only."""
    image, tmpl = _image_args(image, width, height, tmpl)
    th, tw = tmpl.shape
    ys = np.ascontiguousarray(ys, dtype=np.int32)
    xs = np.ascontiguousarray(xs, dtype=np.int32)
    n = ys.size
    res = {k: np.empty(n, dtype=np.uint32) for k in ("sum_i", "sum_isq", "sum_it")}
    res["coef"] = np.empty(n, dtype=np.float32)
    res["coef64"] = np.empty(n, dtype=np.float64)
    st = (lib or _load()).oracle_ncc_u8_points(
        _ptr(image, _u8p), width, height, image.shape[1], _ptr(tmpl, _u8p), tw, th,
        _ptr(ys, _i32p), _ptr(xs, _i32p), n,
        _ptr(res["sum_i"], _u32p), _ptr(res["sum_isq"], _u32p), _ptr(res["sum_it"], _u32p),
        _ptr(res["coef"], _f32p), _ptr(res["coef64"], _f64p), nthreads)
    if st == ORACLE_ERR_U32:
        raise OverflowError("a window sum does not fit in 32 bits")
    if st != ORACLE_OK:
        raise ValueError(f"oracle_ncc_u8_points: bad arguments (status {st})")
    return res


def ncc_peak(coef: np.ndarray, *, lib=None):
    """Best match of a coefficient map: ``(y, x, value)`` of the first entry
    (row-major) holding the largest coefficient."""
    coef = np.ascontiguousarray(coef, dtype=np.float32)
    if coef.ndim != 2 or coef.size == 0:
        raise ValueError("coef must be a non-empty 2D map")
    idx = np.zeros(1, dtype=np.int64)
    val = np.zeros(1, dtype=np.float32)
    st = (lib or _load()).oracle_ncc_peak(_ptr(coef, _f32p), coef.size, _ptr(idx, _i64p), _ptr(val, _f32p))
    if st != ORACLE_OK:
        raise ValueError(f"oracle_ncc_peak: bad arguments (status {st})")
    y, x = divmod(int(idx[0]), coef.shape[1])
    return y, x, float(val[0])


def xcorr_f32(left: np.ndarray, right: np.ndarray, *, with_abs: bool = True, nthreads: int = 0, lib=None):
    """Full cross-correlation of every (left, right) pair, in fp64.

    ``left`` is [n_left, rows, cols] and ``right`` [n_right, rows, cols] fp32.
    Returns ``(out, abs_out)`` of shape [n_left, n_right, 2rows-1, 2cols-1];
    ``abs_out`` (sum of |l*r| over each overlap) is None unless ``with_abs``.
    """
    left = np.ascontiguousarray(left, dtype=np.float32)
    right = np.ascontiguousarray(right, dtype=np.float32)
    if left.ndim == 2:
        left = left[None]
    if right.ndim == 2:
        right = right[None]
    nl, rows, cols = left.shape
    nr = right.shape[0]
    if right.shape[1:] != (rows, cols):
        raise ValueError("left and right matrices must share (rows, cols)")
    shape = (nl, nr, 2 * rows - 1, 2 * cols - 1)
    out = np.empty(shape, dtype=np.float64)
    ab = np.empty(shape, dtype=np.float64) if with_abs else None
    st = (lib or _load()).oracle_xcorr_f32(_ptr(left, _f32p), nl, _ptr(right, _f32p), nr, rows, cols,
                                  _ptr(out, _f64p), _ptr(ab, _f64p), nthreads)
    if st != ORACLE_OK:
        raise ValueError(f"oracle_xcorr_f32: bad arguments (status {st})")
    return out, ab


def xcorr_f32_points(left: np.ndarray, right: np.ndarray, flat_idx, *, nthreads: int = 0, lib=None):
    """Selected outputs (flat indices into the [nl, nr, 2rows-1, 2cols-1] array)."""
    left = np.ascontiguousarray(left, dtype=np.float32)
    right = np.ascontiguousarray(right, dtype=np.float32)
    if left.ndim == 2:
        left = left[None]
    if right.ndim == 2:
        right = right[None]
    nl, rows, cols = left.shape
    nr = right.shape[0]
    flat = np.ascontiguousarray(flat_idx, dtype=np.int64)
    out = np.empty(flat.size, dtype=np.float64)
    ab = np.empty(flat.size, dtype=np.float64)
    st = (lib or _load()).oracle_xcorr_f32_points(_ptr(left, _f32p), nl, _ptr(right, _f32p), nr, rows, cols,
                                         _ptr(flat, _i64p), flat.size, _ptr(out, _f64p), _ptr(ab, _f64p),
                                         nthreads)
    if st != ORACLE_OK:
        raise ValueError(f"oracle_xcorr_f32_points: bad arguments (status {st})")
    return out, ab
