"""MI355X (gfx950) direct sliding-window 2D correlation.

* :func:`ncc_u8` -- 8-bit normalized correlation (template matching).
* :func:`xcorr_f32` -- fp32 full cross-correlation, one-to-one / one-to-many /
  n-to-m.

The computation runs in hand-written HIP kernels behind the C ABI in
``include/xcorr.h`` (``libxcorr_hip.so``, built in-tree by :mod:`.build`).
The torch-facing functions are imported lazily so that the seeded input
generators (:mod:`.inputs`) can be used without torch or a GPU.
"""

__all__ = ["ncc_u8", "xcorr_f32"]


def __getattr__(name):
    if name in ("ncc_u8", "xcorr_f32"):
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
