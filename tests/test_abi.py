"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects invalid arguments before any HIP call.  No compute call
is made here (there is no GPU in this container)."""
import ctypes
import os
import re

import pytest

from cross_correlation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xcorr.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*|size_t)\s*(\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    """Every XC_ constant the header defines has the same value in the binding."""
    found = re.findall(r"^#define (XC_\w+) \(?(-?\d+)\)?", open(HEADER).read(), re.M)
    assert len(found) >= 20
    for name, value in found:
        assert getattr(_lib, name) == int(value), name


def test_status_strings():
    for code in range(0, -9, -1):
        assert _lib.status_str(code) and _lib.status_str(code) != "unknown status"
    assert _lib.status_str(-99) == "unknown status"


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("args,expect", [
    (dict(image=0), _lib.XC_ERR_NULL),
    (dict(tmpl=0), _lib.XC_ERR_NULL),
    (dict(sum_i=0, sum_isq=0, sum_it=0, coef=0), _lib.XC_ERR_NULL),
    (dict(width=0), _lib.XC_ERR_SHAPE),
    (dict(t_height=0), _lib.XC_ERR_SHAPE),
    (dict(t_width=80), _lib.XC_ERR_SHAPE),
    (dict(t_height=70), _lib.XC_ERR_SHAPE),
    (dict(pitch=32), _lib.XC_ERR_SHAPE),
    (dict(width=70000, pitch=70016, height=2, t_width=33028, t_height=2), _lib.XC_ERR_OVERFLOW),
    (dict(image=FAKE + 4), _lib.XC_ERR_ALIGN),
    (dict(pitch=72), _lib.XC_ERR_ALIGN),
    (dict(coef=FAKE + 2), _lib.XC_ERR_ALIGN),
    (dict(variant=42), _lib.XC_ERR_VARIANT),
    (dict(variant=_lib.XC_NCC_MFMA32 + 1), _lib.XC_ERR_VARIANT),
    # the matrix-core tile widths: 128 columns only for templates up to 64 wide
    (dict(t_width=68, width=200, pitch=208, variant=_lib.XC_NCC_MFMA_W2), _lib.XC_ERR_SHAPE),
    (dict(t_width=300, width=400, pitch=400, variant=_lib.XC_NCC_MFMA_W4), _lib.XC_ERR_SHAPE),
    # the 32x32x32 recast: rows up to 65 bytes, templates short enough for its LDS plan
    (dict(t_width=66, width=200, pitch=208, variant=_lib.XC_NCC_MFMA32), _lib.XC_ERR_SHAPE),
    (dict(t_width=64, t_height=351, width=200, height=400, pitch=208, variant=_lib.XC_NCC_MFMA32),
     _lib.XC_ERR_SHAPE),
    (dict(variant=-1), _lib.XC_ERR_VARIANT),
])
def test_ncc_validation(args, expect):
    a = dict(image=FAKE, width=64, height=64, pitch=64, tmpl=FAKE, t_width=8, t_height=8,
             sum_i=FAKE, sum_isq=0, sum_it=0, coef=FAKE, variant=0)
    a.update(args)
    st = _lib.ncc_u8_run(a["image"], a["width"], a["height"], a["pitch"], a["tmpl"], a["t_width"], a["t_height"],
                         a["sum_i"], a["sum_isq"], a["sum_it"], a["coef"], None, a["variant"])
    assert st == expect, _lib.status_str(st)


@pytest.mark.parametrize("args,expect", [
    (dict(peak=0), _lib.XC_ERR_NULL),
    (dict(image=0), _lib.XC_ERR_NULL),
    (dict(peak=FAKE + 4), _lib.XC_ERR_ALIGN),
    (dict(t_width=80), _lib.XC_ERR_SHAPE),
    (dict(variant=42), _lib.XC_ERR_VARIANT),
    (dict(t_width=300, width=400, pitch=400, variant=_lib.XC_NCC_MFMA), _lib.XC_ERR_SHAPE),
])
def test_ncc_peak_validation(args, expect):
    """The best-match entry point: the maps are optional, the peak is not."""
    a = dict(image=FAKE, width=64, height=64, pitch=64, tmpl=FAKE, t_width=8, t_height=8, peak=FAKE, variant=0)
    a.update(args)
    st = _lib.ncc_u8_peak(a["image"], a["width"], a["height"], a["pitch"], a["tmpl"], a["t_width"],
                          a["t_height"], 0, 0, 0, 0, a["peak"], None, a["variant"])
    assert st == expect, _lib.status_str(st)


def test_decode_peak_layout():
    import struct
    raw = struct.pack("<QiifI", 123, 7, 9, 0.5, 0)
    assert _lib.decode_peak(raw) == (7, 9, 0.5)


@pytest.mark.parametrize("args,expect", [
    (dict(left=0), _lib.XC_ERR_NULL),
    (dict(out=0), _lib.XC_ERR_NULL),
    (dict(n_left=0), _lib.XC_ERR_SHAPE),
    (dict(rows=-1), _lib.XC_ERR_SHAPE),
    (dict(rows=40000, cols=40000), _lib.XC_ERR_OVERFLOW),
    (dict(left=FAKE + 8), _lib.XC_ERR_ALIGN),
    (dict(out=FAKE + 2), _lib.XC_ERR_ALIGN),
    (dict(algo=9), _lib.XC_ERR_VARIANT),
    (dict(algo=_lib.XC_XCORR_MFMA + 1), _lib.XC_ERR_VARIANT),
    (dict(rows=8, algo=_lib.XC_XCORR_BLOCKDIAG), _lib.XC_ERR_SHAPE),
    # the fp32 matrix cores: cols a multiple of 4, staging within the plan
    (dict(cols=30, algo=_lib.XC_XCORR_MFMA), _lib.XC_ERR_SHAPE),
    (dict(cols=1000, algo=_lib.XC_XCORR_MFMA), _lib.XC_ERR_SHAPE),
])
def test_xcorr_validation(args, expect):
    a = dict(left=FAKE, n_left=1, right=FAKE, n_right=1, rows=32, cols=32, out=FAKE, algo=0)
    a.update(args)
    st = _lib.xcorr_f32_run(a["left"], a["n_left"], a["right"], a["n_right"], a["rows"], a["cols"], a["out"],
                            None, a["algo"])
    assert st == expect, _lib.status_str(st)


@pytest.mark.parametrize("args,expect", [
    (dict(mode=3), _lib.XC_ERR_VARIANT),
    (dict(mode=-1), _lib.XC_ERR_VARIANT),
    (dict(workspace=0), _lib.XC_ERR_NULL),
    (dict(workspace=FAKE + 8), _lib.XC_ERR_ALIGN),
    (dict(workspace_bytes=100), _lib.XC_ERR_SHAPE),
    (dict(image=FAKE + 4), _lib.XC_ERR_ALIGN),
    (dict(pitch=32), _lib.XC_ERR_SHAPE),
    (dict(t_width=300, t_height=300), _lib.XC_ERR_OVERFLOW),
    (dict(sum_i=0, coef=0), _lib.XC_ERR_NULL),
    (dict(variant=42), _lib.XC_ERR_VARIANT),
    (dict(mode=0, t_width=80), _lib.XC_ERR_SHAPE),
])
def test_ncc_mode_validation(args, expect):
    a = dict(image=FAKE, width=64, height=64, pitch=64, tmpl=FAKE, t_width=8, t_height=8, mode=1, workspace=FAKE,
             workspace_bytes=1 << 20, sum_i=FAKE, coef=FAKE, variant=0)
    a.update(args)
    st = _lib.ncc_u8_run_mode(a["image"], a["width"], a["height"], a["pitch"], a["tmpl"], a["t_width"],
                              a["t_height"], a["mode"], a["workspace"], a["workspace_bytes"], a["sum_i"], 0, 0,
                              a["coef"], None, a["variant"])
    assert st == expect, _lib.status_str(st)


def test_ncc_mode_workspace_sizes():
    """Workspace bytes: the padded image, rows of a 16-byte multiple pitch."""
    for (w, h, tw, th, mode, expect) in ((64, 64, 8, 8, 0, 0),
                                         (64, 64, 8, 8, 1, (64 + 7) * ((64 + 7 + 15) // 16 * 16)),
                                         (64, 64, 8, 8, 2, (64 + 14) * ((64 + 14 + 15) // 16 * 16)),
                                         (10, 12, 30, 20, 2, (12 + 38) * ((10 + 58 + 15) // 16 * 16))):
        st, n = _lib.ncc_u8_mode_workspace(w, h, tw, th, mode)
        assert st == 0 and n == expect, (w, h, tw, th, mode, n)
    assert _lib.ncc_u8_mode_workspace(64, 64, 80, 8, 0)[0] == _lib.XC_ERR_SHAPE
    assert _lib.ncc_u8_mode_workspace(64, 64, 80, 8, 1)[0] == 0  # same mode: larger templates allowed
    assert _lib.ncc_u8_mode_workspace(64, 64, 8, 8, 5)[0] == _lib.XC_ERR_VARIANT
    assert _lib.ncc_mode_shape(20, 10, 5, 3, _lib.XC_NCC_MODE_FULL) == (12, 24)


def test_ncc_auto_variant_choice():
    """The automatic kernel choice, queried without a launch (no device here,
    so the rule uses the MI355X's 256 compute units)."""
    M, C1, ILP = _lib.XC_NCC_MFMA, _lib.XC_NCC_DOT4_C1, _lib.XC_NCC_DOT4_ILP
    for (w, h, tw, th, expect) in (
            (1920, 1080, 64, 64, M),    # the headline workload: 512+ template pixels
            (1920, 1080, 4, 4, M),      # a million outputs
            (1280, 720, 16, 16, M),     # 96+ pixels and 400K+ outputs
            (1280, 720, 8, 8, ILP),     # 225 big packed-byte tiles, too much work for one-per-thread
            (1280, 720, 7, 7, M),       # the same with an unaligned width
            (768, 768, 8, 8, C1),       # 144 big packed-byte tiles, 37K word-workgroups
            (1600, 600, 4, 4, ILP),     # 266 big packed-byte tiles fill the chip
            (256, 256, 16, 16, C1),     # small image, aligned template
            (640, 480, 8, 8, C1),
            (640, 480, 16, 16, M),      # one-per-thread grid x words over 192 per CU
            (256, 256, 24, 24, C1),     # 144 words, grid x words within 180 per CU
            (300, 300, 24, 24, M),      # 144 words over 180 per CU
            (256, 256, 32, 32, M),      # 256 words
            (384, 384, 6, 6, C1),       # unaligned, 12 words
            (400, 300, 10, 10, M),      # unaligned, 30 words
            (64, 64, 64, 64, M),        # one output, 4096 pixels
            (300, 40, 257, 7, ILP)):    # a template too wide for the matrix cores
        st, v = _lib.ncc_u8_auto_variant(w, h, tw, th)
        assert st == 0 and v == expect, (w, h, tw, th, v)
    assert _lib.ncc_u8_auto_variant(10, 10, 20, 3)[0] == _lib.XC_ERR_SHAPE
    assert _lib.ncc_u8_auto_variant(600, 600, 300, 300)[0] == _lib.XC_ERR_OVERFLOW
    # the output-count limit, 2^31 - 1 windows: 2045 x 1,050,114 passes, one more row does not
    assert _lib.ncc_u8_auto_variant(2048, 1050117, 4, 4)[0] == 0
    assert _lib.ncc_u8_auto_variant(2048, 1050118, 4, 4)[0] == _lib.XC_ERR_OVERFLOW
    assert _lib.load().ncc_u8_auto_variant(64, 64, 8, 8, None) == _lib.XC_ERR_NULL
