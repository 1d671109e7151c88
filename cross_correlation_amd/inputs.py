"""Seeded synthetic inputs for the two correlation forms.

This module only *makes data*: it draws pixels and matrix entries from
``numpy.random.default_rng(seed)`` (PCG64) and cuts templates out of images.
It holds none of the correlation arithmetic, so both the CPU oracle and the
GPU path can consume the same inputs without sharing any method code.

The shapes follow the workloads the pages discuss:

* u8 normalized correlation (The CUDA Handbook, section 15.5): an 8-bit
  grayscale image and a template whose width is a multiple of four, cut from
  the image so that the best match is known.
* fp32 full cross-correlation of matrix pairs (JPDC 2023 artifact README,
  the warp-shuffle / multi-matrix kernel overview): one-to-one, one-to-many
  and n-to-m groupings of equally sized matrices with entries in [-1, 1).

The pages name no dataset; every input here is synthetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "NccCase",
    "XcorrCase",
    "u8_uniform",
    "f32_uniform",
    "gradient_image",
    "ncc_case",
    "xcorr_case",
    "NCC_WORKLOADS",
    "XCORR_WORKLOADS",
    "pitch_for",
]


def pitch_for(width: int, align: int = 16) -> int:
    """Smallest row pitch >= width that is a multiple of ``align`` bytes."""
    return (width + align - 1) // align * align


def u8_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform bytes in [0, 255]."""
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def f32_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform fp32 in [-1, 1) on the 2^-23 grid.

    Every value k / 2^23 - 1 with integer k in [0, 2^24) is exactly
    representable in fp32, so the fp32 and fp64 views of an input agree.
    """
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) / float(1 << 23) - 1.0).astype(np.float32)


def gradient_image(rng: np.random.Generator, height: int, width: int) -> np.ndarray:
    """Uniform bytes averaged with a smooth diagonal ramp.

    I = (U + G) >> 1 with U uniform in [0, 255] and
    G[y][x] = floor(255 * (x + y) / (width + height - 2)); the result stays in
    [0, 255] without clipping.
    """
    u = u8_uniform(rng, (height, width)).astype(np.uint16)
    yy, xx = np.mgrid[0:height, 0:width]
    denom = max(width + height - 2, 1)
    g = (255 * (xx + yy)) // denom
    return ((u + g.astype(np.uint16)) >> 1).astype(np.uint8)


@dataclass
class NccCase:
    """An 8-bit image (row pitch = ``pitch`` bytes) plus a template."""

    name: str
    image: np.ndarray  # (height, pitch) uint8, columns >= width are padding
    width: int
    height: int
    tmpl: np.ndarray  # (t_height, t_width) uint8, dense
    cut: tuple[int, int] | None  # (oy, ox) where the template was cut, if any

    @property
    def pitch(self) -> int:
        return int(self.image.shape[1])

    @property
    def t_height(self) -> int:
        return int(self.tmpl.shape[0])

    @property
    def t_width(self) -> int:
        return int(self.tmpl.shape[1])

    @property
    def out_shape(self) -> tuple[int, int]:
        return (self.height - self.t_height + 1, self.width - self.t_width + 1)

    def pixels(self) -> np.ndarray:
        """The (height, width) view without row padding."""
        return self.image[:, : self.width]


@dataclass
class XcorrCase:
    """Left matrices [n_left, rows, cols] and right matrices [n_right, rows, cols]."""

    name: str
    left: np.ndarray
    right: np.ndarray

    @property
    def rows(self) -> int:
        return int(self.left.shape[1])

    @property
    def cols(self) -> int:
        return int(self.left.shape[2])

    @property
    def out_shape(self) -> tuple[int, int, int, int]:
        return (self.left.shape[0], self.right.shape[0], 2 * self.rows - 1, 2 * self.cols - 1)


def _padded(img: np.ndarray, pitch: int) -> np.ndarray:
    h, w = img.shape
    out = np.zeros((h, pitch), dtype=np.uint8)
    out[:, :w] = img
    return out


def ncc_case(
    name: str,
    seed: int,
    height: int,
    width: int,
    t_height: int,
    t_width: int,
    *,
    image_kind: str = "uniform",
    cut: bool = True,
    pitch: int | None = None,
) -> NccCase:
    """Image plus template.

    Draw order: the image, then (when ``cut``) the cut offset (oy, ox) as two
    ``rng.integers`` calls; otherwise an independent uniform template.
    """
    rng = np.random.default_rng(seed)
    if image_kind == "uniform":
        img = u8_uniform(rng, (height, width))
    elif image_kind == "gradient":
        img = gradient_image(rng, height, width)
    else:
        raise ValueError(f"unknown image kind {image_kind!r}")
    out_h, out_w = height - t_height + 1, width - t_width + 1
    if cut:
        oy = int(rng.integers(out_h))
        ox = int(rng.integers(out_w))
        tmpl = np.ascontiguousarray(img[oy : oy + t_height, ox : ox + t_width])
        where = (oy, ox)
    else:
        tmpl = u8_uniform(rng, (t_height, t_width))
        where = None
    p = pitch_for(width) if pitch is None else pitch
    return NccCase(name, _padded(img, p), width, height, tmpl, where)


def xcorr_case(name: str, seed: int, n_left: int, n_right: int, rows: int, cols: int) -> XcorrCase:
    """Draw order: all left matrices, then all right matrices."""
    rng = np.random.default_rng(seed)
    left = f32_uniform(rng, (n_left, rows, cols))
    right = f32_uniform(rng, (n_right, rows, cols))
    return XcorrCase(name, left, right)


# The five workloads: two u8 NCC images and three fp32 groupings.
NCC_WORKLOADS = {
    "ncc_256x256_t16": dict(seed=1, height=256, width=256, t_height=16, t_width=16, image_kind="uniform"),
    "ncc_1920x1080_t64": dict(seed=2, height=1080, width=1920, t_height=64, t_width=64, image_kind="gradient"),
}

XCORR_WORKLOADS = {
    "xcorr_1to1_256": dict(seed=3, n_left=1, n_right=1, rows=256, cols=256),
    "xcorr_1to64_64": dict(seed=4, n_left=1, n_right=64, rows=64, cols=64),
    "xcorr_8to16_32": dict(seed=5, n_left=8, n_right=16, rows=32, cols=32),
}


def workload(name: str):
    """Build one of the named workloads."""
    if name in NCC_WORKLOADS:
        return ncc_case(name, **NCC_WORKLOADS[name])
    if name in XCORR_WORKLOADS:
        return xcorr_case(name, **XCORR_WORKLOADS[name])
    raise KeyError(name)
