"""ncc_u8_run_mode_noalloc, the same and full output modes without a
caller-owned workspace (the padded image goes to the library's static device
scratch), called through the C ABI: its outputs equal ncc_u8_run_mode's with
a workspace bit for bit, on two calls in a row (the second with a smaller
image, so stale scratch contents from the first must not leak into it), the
padded image over the scratch size is refused, and valid mode needs no
scratch.  Each case is printed before it touches the GPU."""
import numpy as np
import pytest
import torch

from cross_correlation_amd import _lib
from cross_correlation_amd.inputs import ncc_case

import _gpu

pytestmark = pytest.mark.gpu

MAPS = ("sum_i", "sum_isq", "sum_it", "coef")


def _outs(oh, ow):
    return {k: torch.full((oh, ow), -1, dtype=torch.float32 if k == "coef" else torch.int32, device="cuda")
            for k in MAPS}


def _call(fn, case, mode, outs, extra=()):
    img, tm = _gpu.to_dev(case.image), _gpu.to_dev(case.tmpl)
    p = [outs[k].data_ptr() for k in MAPS]
    st = fn(img.data_ptr(), case.width, case.height, case.pitch, tm.data_ptr(), case.t_width, case.t_height, mode,
            *extra, *p, stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


def _with_workspace(case, mode):
    st, nbytes = _lib.ncc_u8_mode_workspace(case.width, case.height, case.t_width, case.t_height, mode)
    assert st == 0
    oh, ow = _lib.ncc_mode_shape(case.width, case.height, case.t_width, case.t_height, mode)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    outs = _outs(oh, ow)
    assert _call(_lib.ncc_u8_run_mode, case, mode, outs, (ws.data_ptr(), nbytes)) == 0
    return {k: v.cpu().numpy() for k, v in outs.items()}


def _no_alloc(case, mode):
    oh, ow = _lib.ncc_mode_shape(case.width, case.height, case.t_width, case.t_height, mode)
    outs = _outs(oh, ow)
    assert _call(_lib.ncc_u8_run_mode_noalloc, case, mode, outs) == 0
    return {k: v.cpu().numpy() for k, v in outs.items()}


@pytest.mark.parametrize("mode", [_lib.XC_NCC_MODE_SAME, _lib.XC_NCC_MODE_FULL, _lib.XC_NCC_MODE_VALID])
def test_no_alloc_matches_workspace_two_calls(mode):
    big = ncc_case("na_big", 1201, 1080, 1920, 64, 64, image_kind="gradient", cut=True)
    small = ncc_case("na_small", 1202, 300, 411, 13, 10, cut=True)
    for case in (big, small):
        _gpu.log(f"no-alloc mode {mode} {case.height}x{case.width} t{case.t_height}x{case.t_width}")
        a = _no_alloc(case, mode)
        b = _with_workspace(case, mode)
        for k in MAPS:
            assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (case.name, k)


def test_no_alloc_rejects_padded_image_over_scratch():
    # 4000 x 4000 in full mode with a 64 x 64 template: 4063 rows of 4064 bytes > 16 MiB
    st, nbytes = _lib.ncc_u8_mode_workspace(4000, 4000, 64, 64, _lib.XC_NCC_MODE_FULL)
    assert st == 0 and nbytes > _lib.XC_NCC_MODE_SCRATCH_BYTES
    _gpu.log("no-alloc over the scratch size")
    img = torch.zeros((4000, 4000), dtype=torch.uint8, device="cuda")
    tm = torch.zeros((64, 64), dtype=torch.uint8, device="cuda")
    out = torch.zeros((4063, 4063), dtype=torch.float32, device="cuda")
    st = _lib.ncc_u8_run_mode_noalloc(img.data_ptr(), 4000, 4000, 4000, tm.data_ptr(), 64, 64,
                                      _lib.XC_NCC_MODE_FULL, 0, 0, 0, out.data_ptr())
    assert st == _lib.XC_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 0).all())
