"""The no-allocation entry point (twl_ternary_linear_noalloc) against the
workspace entry point (twl_ternary_linear_ex) through the C ABI: the same
kernels, so the outputs must be equal bit for bit.  Each case makes two calls
in a row on the library's per-GPU scratch, the second with a smaller input,
on plans that need K-split scratch (GEMM split-K, the decode kernels' K
slices); one case also checks acc against the CPU oracle.  A shape whose plan
needs more than the scratch holds is refused with TWL_ESHAPE.
"""
import ctypes

import numpy as np
import pytest

import oracle.twl_oracle as O
import workloads as W
from tests.gpu_helpers import announce, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def twl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_linear_block_amd as m
    m.library()
    return m


def _layer(twl, M, N, K, seed):
    L = W.make_layer(seed, M, K, N, codes="sparse40")
    x_i8, a_scale = O.rotate_quant_act(L.x_bits, L.sign)
    packed, q, smax = twl.pack_ternary(dev(L.code), dev(L.s_bits.view(np.int16)))
    return L, x_i8, a_scale, packed, q, smax


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call_ex(twl, lib, xi, sc, packed, q, smax, out, kind, path):
    M, K = xi.shape
    N = q.shape[0]
    need = twl.workspace_bytes(M, N, K)
    ws = torch.full((max(need, 16),), 0x5A, dtype=torch.uint8, device="cuda")
    st = lib.twl_ternary_linear_ex(_ptr(xi), _ptr(sc), _ptr(packed), _ptr(q), _ptr(smax), M, N, K, _ptr(out),
                                   kind, path, _ptr(ws), ws.numel(), None)
    assert st == 0, lib.twl_last_error()
    torch.cuda.synchronize()
    return host(out.view(torch.int16) if out.dtype == torch.bfloat16 else out).copy()


def _call_noalloc(lib, xi, sc, packed, q, smax, out, kind, path):
    M, K = xi.shape
    N = q.shape[0]
    st = lib.twl_ternary_linear_noalloc(_ptr(xi), _ptr(sc), _ptr(packed), _ptr(q), _ptr(smax), M, N, K,
                                        _ptr(out), kind, path, None)
    assert st == 0, lib.twl_last_error()
    torch.cuda.synchronize()
    return host(out.view(torch.int16) if out.dtype == torch.bfloat16 else out).copy()


# (first shape, second smaller shape, path): each first shape's plan uses
# the K-split scratch
CASES = [
    ((256, 5120, 17408), (100, 3000, 17408), 1),   # GEMM with split-K partial tiles
    ((9, 200, 20480), (3, 130, 10240), 4),         # K-split matrix-core decode + slice reduce
    ((1, 129, 32768), (1, 65, 16384), 3),          # dot4 decode, K slices + slice reduce
]


@pytest.mark.parametrize("first,second,path", CASES)
def test_noalloc_equals_workspace_entry_point(twl, first, second, path):
    lib = twl.library()
    for i, (M, N, K) in enumerate((first, second)):
        need = twl.workspace_bytes(M, N, K)
        plan = twl.plan_info(M, N, K, path)
        if i == 0:
            assert plan["workspace_bytes"] > 0, plan
        assert plan["workspace_bytes"] <= twl._lib.NOALLOC_SCRATCH_BYTES
        L, x_i8, a_scale, packed, q, smax = _layer(twl, M, N, K, 9000 + M + N + i)
        xi, sc = dev(x_i8), dev(a_scale)
        for kind, dtype in ((1, torch.int32), (0, torch.float32), (2, torch.bfloat16)):
            announce(f"noalloc vs ex M={M} N={N} K={K} path={path} kind={kind} need={need}")
            a = _call_ex(twl, lib, xi, sc, packed, q, smax, torch.empty((M, N), dtype=dtype, device="cuda"),
                         kind, path)
            b = _call_noalloc(lib, xi, sc, packed, q, smax,
                              torch.full((M, N), 7, dtype=dtype, device="cuda"), kind, path)
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"kind {kind}: outputs differ"
            if kind == 1 and i == 0:
                assert np.array_equal(b, O.linear_acc(x_i8, L.code, O.decompose_scales(L.s_bits)[0]))


def test_noalloc_binding_and_refusal(twl):
    lib = twl.library()
    # the binding writes into the caller's tensor
    M, N, K = 40, 300, 32768
    L, x_i8, a_scale, packed, q, smax = _layer(twl, M, N, K, 9100)
    xi, sc = dev(x_i8), dev(a_scale)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    announce(f"noalloc binding M={M} N={N} K={K}")
    twl.ternary_linear_noalloc(xi, sc, packed, q, smax, y)
    ref = twl.ternary_linear(xi, sc, packed, q, smax)
    assert np.array_equal(host(y).view(np.uint32), host(ref).view(np.uint32))
    # a plan that needs more than the scratch holds is refused before any launch
    big = None
    for shape in ((512, 4096, 65536), (256, 8192, 65536), (512, 8192, 65536), (1024, 4096, 65536),
                  (384, 6144, 65536), (256, 16384, 65536)):
        if twl.workspace_bytes(*shape) > twl._lib.NOALLOC_SCRATCH_BYTES:
            big = shape
            break
    assert big is not None, "no candidate shape needs more than the scratch"
    M, N, K = big
    fake = ctypes.c_void_p(0x10000)
    st = lib.twl_ternary_linear_noalloc(fake, fake, fake, fake, fake, M, N, K, fake, 0, 0, None)
    assert st == 2, st
    assert b"no-allocation scratch" in lib.twl_last_error()
