"""Host-side checks of the C ABI that need no GPU: the built library loads,
exports every function include/twl.h declares, and rejects bad arguments on
the host (shape, null pointer, alignment) before touching the device.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twl.h")

twl = pytest.importorskip("ternary_weight_linear_block_amd")
from ternary_weight_linear_block_amd import _lib  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(twl_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtwl.so is not built; run `python -m ternary_weight_linear_block_amd.build`")
    return _lib.load()


def test_header_declares_the_three_operations():
    names = _declared_functions()
    for n in ("twl_rotate_quant_act", "twl_pack_ternary", "twl_ternary_linear"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    # the binding's prototypes cover exactly the header's functions
    assert sorted(s[0] for s in _lib.SIGNATURES) == names


def test_abi_version(lib):
    assert lib.twl_abi_version() == 3


FAKE = 0x10000   # 16-byte aligned, never dereferenced: every call below fails host validation


@pytest.mark.parametrize("K", [0, 1000, 1024 + 128, 65536 + 1024])
def test_rotate_rejects_bad_k(lib, K):
    st = lib.twl_rotate_quant_act(FAKE, FAKE, 4, K, FAKE, FAKE, None)
    assert st == 2  # TWL_ESHAPE
    assert b"K=" in lib.twl_last_error()


def test_rotate_rejects_null_and_misaligned(lib):
    assert lib.twl_rotate_quant_act(None, FAKE, 4, 1024, FAKE, FAKE, None) == 1
    assert b"x is NULL" in lib.twl_last_error()
    assert lib.twl_rotate_quant_act(FAKE + 2, FAKE, 4, 1024, FAKE, FAKE, None) == 3
    assert lib.twl_rotate_quant_act(FAKE, FAKE, -1, 1024, FAKE, FAKE, None) == 1


def test_fused_activation_rejects_bad_args(lib):
    f = lib.twl_silu_mul_rotate_quant_act
    assert f(FAKE, FAKE, 4, 1000, FAKE, FAKE, None) == 2
    assert f(None, FAKE, 4, 1024, FAKE, FAKE, None) == 1
    assert f(FAKE + 2, FAKE, 4, 1024, FAKE, FAKE, None) == 3
    assert f(None, None, 0, 1024, None, None, None) == 0


def test_rotate_quant_linear_rejects_bad_args(lib):
    f = lib.twl_rotate_quant_linear
    P = FAKE

    def call(x=P, sign=P, packed=P, q=P, smax=P, M=4, N=64, K=1024, silu=0, x_i8=P, a_scale=P,
             out=P, kind=0):
        return f(x, sign, packed, q, smax, M, N, K, silu, x_i8, a_scale, out, kind, None, 0, None)

    assert call(K=1000) == 2 and b"K=" in lib.twl_last_error()
    assert call(silu=2) == 1 and b"silu" in lib.twl_last_error()
    assert call(kind=5) == 1
    assert call(M=-1) == 1
    assert call(x=None) == 1 and b"x is NULL" in lib.twl_last_error()
    assert call(sign=P + 2) == 3
    assert call(x_i8=None) == 1
    assert call(a_scale=None) == 1
    assert call(packed=None) == 1 and b"packed is NULL" in lib.twl_last_error()
    assert call(out=None) == 1
    assert call(smax=None) == 1
    # M = 0 is a no-op; N = 0 needs only the rotation's buffers (it then fails
    # later, on the device query, which this host has not: not a validation error)
    assert call(x=None, sign=None, packed=None, q=None, smax=None, M=0, x_i8=None, a_scale=None,
                out=None) == 0
    assert call(packed=None, q=None, smax=None, out=None, N=0) not in (1, 2, 3)
    # the raw accumulators need no smax
    assert call(smax=None, kind=1) not in (1, 2, 3)
    fused = lib.twl_rotate_quant_linear_fused
    assert fused(4, 64, 1000) == -2
    assert fused(-1, 64, 1024) == -1


def test_pack_rejects_bad_args(lib):
    assert lib.twl_pack_ternary(FAKE, FAKE, 8, 1000, FAKE, FAKE, FAKE, None, None) == 2
    assert lib.twl_pack_ternary(FAKE, None, 8, 1024, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.twl_pack_ternary(FAKE, FAKE, 8, 1024, FAKE, FAKE, FAKE, FAKE + 2, None) == 3


def test_linear_rejects_bad_args(lib):
    ex = lib.twl_ternary_linear_ex
    # unknown paths
    for path in (-1, 5, 7):
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 1024, FAKE, 0, path, None, 0, None) == 1
    # unknown output kinds
    for kind in (-1, 3):
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 1024, FAKE, kind, 0, None, 0, None) == 1
    # bf16 y needs a_scale and smax too
    assert ex(FAKE, FAKE, FAKE, FAKE, None, 4, 4, 1024, FAKE, 2, 0, None, 0, None) == 1
    # the decode paths (automatic, dot4, MFMA) beyond their batch limit
    for path in (2, 3, 4):
        assert ex(FAKE, FAKE, FAKE, FAKE, FAKE, 25, 4, 1024, FAKE, 0, path, None, 0, None) == 2
    # y output needs a_scale and smax; acc output does not
    assert ex(FAKE, None, FAKE, FAKE, FAKE, 4, 4, 1024, FAKE, 0, 0, None, 0, None) == 1
    assert ex(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 3072 + 64, FAKE, 1, 0, None, 0, None) == 2
    assert lib.twl_ternary_linear(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 1024, FAKE + 8, None, 0, None) == 3


def test_empty_shapes_enqueue_nothing(lib):
    # M = 0 or N = 0 return OK before any device query
    assert lib.twl_rotate_quant_act(None, None, 0, 1024, None, None, None) == 0
    assert lib.twl_pack_ternary(None, None, 0, 1024, None, None, None, None, None) == 0
    assert lib.twl_ternary_linear(None, None, None, None, None, 0, 5, 1024, None, None, 0, None) == 0
    assert lib.twl_ternary_linear(None, None, None, None, None, 5, 0, 1024, None, None, 0, None) == 0
    assert lib.twl_last_error() == b""


def test_peaks_library_exports_its_microbenchmarks():
    # libtwl_peaks.so: the microbenchmark kernels bench.py times for the
    # measured peaks (not part of the ternary-linear ABI); loading only
    from ternary_weight_linear_block_amd.build import PEAKS_LIB_PATH
    if not os.path.exists(PEAKS_LIB_PATH):
        pytest.skip("libtwl_peaks.so not built")
    lib = ctypes.CDLL(PEAKS_LIB_PATH)
    for name in ("twl_peak_mfma_i8", "twl_peak_read", "twl_peak_dot4", "twl_peak_mix_i8"):
        assert hasattr(lib, name), name
