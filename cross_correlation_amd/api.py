"""Torch-facing wrappers: device memory and streams from PyTorch, every
computation in the HIP library (``_lib``).  The u32 sums come back in int32
tensors holding the 32-bit patterns (``.view(torch.uint32)`` or
``numpy().view(np.uint32)`` recovers the unsigned values).
"""
from __future__ import annotations

import torch

from . import _lib


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _device_u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 CUDA tensor")
    return t


_SUM_DTYPES = (torch.int32, torch.uint32)


def _check_out(t, name: str, numel: int, dtypes, device: torch.device) -> None:
    """A caller-supplied output the kernels write densely: it must be a
    contiguous tensor of one of ``dtypes`` on ``device`` holding exactly
    ``numel`` elements, else ValueError (checked before any launch, so a
    wrong buffer never receives out-of-bounds writes)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the output has {numel}")


def _check_maps(out: dict, oh: int, ow: int, device: torch.device) -> None:
    """Every map in ``out`` (sum_i, sum_isq, sum_it as 32-bit integers, coef
    as float32) must be a dense [oh, ow] buffer on ``device``."""
    unknown = set(out) - {"sum_i", "sum_isq", "sum_it", "coef"}
    if unknown:
        raise ValueError(f"unknown outputs {sorted(unknown)}")
    n = max(oh, 0) * max(ow, 0)
    for k, t in out.items():
        _check_out(t, f"out[{k!r}]", n, (torch.float32,) if k == "coef" else _SUM_DTYPES, device)


def _check_bytes(t, name: str, nbytes: int, device: torch.device) -> None:
    """A caller-supplied device buffer of at least ``nbytes`` contiguous bytes on ``device``."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} are needed")


def ncc_u8(image: torch.Tensor, tmpl: torch.Tensor, *, width: int | None = None,
           outputs=("sum_i", "sum_isq", "sum_it", "coef"), variant: int = _lib.XC_NCC_AUTO,
           out: dict | None = None, stream=None) -> dict:
    """Valid-mode u8 normalized correlation.

    ``image`` is a [height, pitch] uint8 CUDA tensor (rows contiguous, pitch a
    multiple of 16 bytes, only the first ``width`` columns are pixels);
    ``tmpl`` a dense [t_height, t_width] uint8 CUDA tensor (any width).  Returns a dict of
    the requested outputs, each [out_h, out_w]; pass ``out`` to reuse buffers.
    """
    _device_u8(image, "image")
    _device_u8(tmpl, "tmpl")
    if image.dim() != 2 or image.stride(1) != 1 or tmpl.dim() != 2 or not tmpl.is_contiguous():
        raise ValueError("image must be 2D with unit column stride; tmpl must be 2D contiguous")
    height, pitch = image.shape[0], image.stride(0)
    width = image.shape[1] if width is None else width
    th, tw = tmpl.shape
    oh, ow = height - th + 1, width - tw + 1
    if out is None:
        out = {}
        for k in outputs:
            dt = torch.float32 if k == "coef" else torch.int32
            out[k] = torch.empty((max(oh, 0), max(ow, 0)), dtype=dt, device=image.device)
    else:
        _check_maps(out, oh, ow, image.device)
    ptr = {k: (out[k].data_ptr() if k in out else 0) for k in ("sum_i", "sum_isq", "sum_it", "coef")}
    st = _lib.ncc_u8_run(image.data_ptr(), width, height, pitch, tmpl.data_ptr(), tw, th,
                         ptr["sum_i"], ptr["sum_isq"], ptr["sum_it"], ptr["coef"],
                         _stream_handle(stream), variant)
    _lib.check(st, "ncc_u8_run")
    return out


def ncc_u8_peak(image: torch.Tensor, tmpl: torch.Tensor, *, width: int | None = None, outputs=(),
                variant: int = _lib.XC_NCC_AUTO, out: dict | None = None, peak: torch.Tensor | None = None,
                stream=None) -> dict:
    """Best match of the valid-mode u8 normalized correlation.

    Same inputs as :func:`ncc_u8`; ``outputs`` (default none) selects maps to
    return as well.  The result dict holds those maps and ``"peak"``, the
    device tensor of the xc_ncc_peak (decode it with
    ``_lib.decode_peak(peak.cpu().numpy().tobytes())`` after synchronizing).
    """
    _device_u8(image, "image")
    _device_u8(tmpl, "tmpl")
    if image.dim() != 2 or image.stride(1) != 1 or tmpl.dim() != 2 or not tmpl.is_contiguous():
        raise ValueError("image must be 2D with unit column stride; tmpl must be 2D contiguous")
    height, pitch = image.shape[0], image.stride(0)
    width = image.shape[1] if width is None else width
    th, tw = tmpl.shape
    oh, ow = height - th + 1, width - tw + 1
    if out is None:
        out = {}
        for k in outputs:
            dt = torch.float32 if k == "coef" else torch.int32
            out[k] = torch.empty((max(oh, 0), max(ow, 0)), dtype=dt, device=image.device)
    else:
        _check_maps(out, oh, ow, image.device)
    if peak is None:
        peak = torch.empty(_lib.PEAK_BYTES // 8, dtype=torch.int64, device=image.device)
    else:
        _check_bytes(peak, "peak", _lib.PEAK_BYTES, image.device)
    ptr = {k: (out[k].data_ptr() if k in out else 0) for k in ("sum_i", "sum_isq", "sum_it", "coef")}
    st = _lib.ncc_u8_peak(image.data_ptr(), width, height, pitch, tmpl.data_ptr(), tw, th,
                          ptr["sum_i"], ptr["sum_isq"], ptr["sum_it"], ptr["coef"], peak.data_ptr(),
                          _stream_handle(stream), variant)
    _lib.check(st, "ncc_u8_peak")
    res = dict(out)
    res["peak"] = peak
    return res


def ncc_u8_mode(image: torch.Tensor, tmpl: torch.Tensor, mode: int, *, width: int | None = None,
                outputs=("sum_i", "sum_isq", "sum_it", "coef"), variant: int = _lib.XC_NCC_AUTO,
                out: dict | None = None, workspace: torch.Tensor | None = None, stream=None) -> dict:
    """u8 normalized correlation in an output mode (``_lib.XC_NCC_MODE_*``):
    valid, same or full, the last two over the image with zero borders.

    Same inputs as :func:`ncc_u8`; ``workspace`` (a uint8 CUDA tensor of at
    least ``_lib.ncc_u8_mode_workspace(...)`` bytes) is allocated here when
    not given.  Returns the requested outputs, each [out_h, out_w].
    """
    _device_u8(image, "image")
    _device_u8(tmpl, "tmpl")
    if image.dim() != 2 or image.stride(1) != 1 or tmpl.dim() != 2 or not tmpl.is_contiguous():
        raise ValueError("image must be 2D with unit column stride; tmpl must be 2D contiguous")
    height, pitch = image.shape[0], image.stride(0)
    width = image.shape[1] if width is None else width
    th, tw = tmpl.shape
    st, nbytes = _lib.ncc_u8_mode_workspace(width, height, tw, th, mode)
    _lib.check(st, "ncc_u8_mode_workspace")
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=image.device)
    elif workspace is not None:
        _check_bytes(workspace, "workspace", nbytes, image.device)
    oh, ow = _lib.ncc_mode_shape(width, height, tw, th, mode)
    if out is None:
        out = {}
        for k in outputs:
            dt = torch.float32 if k == "coef" else torch.int32
            out[k] = torch.empty((max(oh, 0), max(ow, 0)), dtype=dt, device=image.device)
    else:
        _check_maps(out, oh, ow, image.device)
    ptr = {k: (out[k].data_ptr() if k in out else 0) for k in ("sum_i", "sum_isq", "sum_it", "coef")}
    ws_ptr = workspace.data_ptr() if workspace is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _lib.ncc_u8_run_mode(image.data_ptr(), width, height, pitch, tmpl.data_ptr(), tw, th, mode, ws_ptr,
                              ws_bytes, ptr["sum_i"], ptr["sum_isq"], ptr["sum_it"], ptr["coef"],
                              _stream_handle(stream), variant)
    _lib.check(st, "ncc_u8_run_mode")
    return out


def xcorr_f32(left: torch.Tensor, right: torch.Tensor, *, algo: int = _lib.XC_XCORR_AUTO,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Full cross-correlation of every (left, right) pair.

    ``left`` [n_left, rows, cols] and ``right`` [n_right, rows, cols] are
    contiguous float32 CUDA tensors (2D inputs are taken as one matrix).
    Returns [n_left, n_right, 2*rows-1, 2*cols-1] float32.
    """
    if left.dim() == 2:
        left = left.unsqueeze(0)
    if right.dim() == 2:
        right = right.unsqueeze(0)
    for t, n in ((left, "left"), (right, "right")):
        if t.device.type != "cuda" or t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous float32 CUDA tensor")
    nl, rows, cols = left.shape
    nr = right.shape[0]
    if tuple(right.shape[1:]) != (rows, cols):
        raise ValueError("left and right matrices must share (rows, cols)")
    if right.device != left.device:
        raise ValueError(f"right is on {right.device}, left on {left.device}")
    if out is None:
        out = torch.empty((nl, nr, 2 * rows - 1, 2 * cols - 1), dtype=torch.float32, device=left.device)
    else:
        _check_out(out, "out", nl * nr * (2 * rows - 1) * (2 * cols - 1), (torch.float32,), left.device)
    st = _lib.xcorr_f32_run(left.data_ptr(), nl, right.data_ptr(), nr, rows, cols, out.data_ptr(),
                            _stream_handle(stream), algo)
    _lib.check(st, "xcorr_f32_run")
    return out
