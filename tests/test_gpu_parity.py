"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for x_i8, a_scale, packed, q, smax and the int32
accumulators; fp32 y within 1e-5 relative, element by element.
"""
import numpy as np
import pytest

import oracle.twl_oracle as O
import workloads as W
from tests.gpu_helpers import announce, dev, gpu_linear, gpu_pack, gpu_rotq, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

Y_RTOL = 1e-5


@pytest.fixture(scope="module")
def twl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_linear_block_amd as m
    m.library()  # raises if libtwl.so is missing: no fallback exists
    return m


def _oracle_layer(layer):
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax = O.pack_ternary(layer.code, layer.s_bits)
    return x_i8, a_scale, packed, q, smax


def _check_rotq(twl, x_bits, sign, label):
    announce(f"rotate_quant_act {label} M={x_bits.shape[0]} K={x_bits.shape[1]}")
    gx, gs = gpu_rotq(twl, x_bits, sign)
    ox, os_ = O.rotate_quant_act(x_bits, sign)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{label}: a_scale differs"
    bad = np.argwhere(gx != ox)
    assert bad.size == 0, f"{label}: {len(bad)} x_i8 mismatches, first {bad[:5].tolist()}"
    return ox, os_


def _check_pack(twl, code, s_bits, label):
    announce(f"pack_ternary {label} N={code.shape[0]} K={code.shape[1]}")
    packed, q, smax = gpu_pack(twl, code, s_bits)
    op, oq, osm = O.pack_ternary(code, s_bits)
    assert np.array_equal(host(packed).reshape(-1), op.reshape(-1)), f"{label}: packed differs"
    assert np.array_equal(host(q), oq), f"{label}: q differs"
    assert np.array_equal(host(smax).view(np.uint32), osm.view(np.uint32)), f"{label}: smax differs"
    return packed, q, smax, oq, osm


def _check_linear(twl, x_i8, a_scale, packed, q, smax, code, oq, osm, path, label):
    pname = {0: "auto", 1: "gemm", 2: "gemv", 3: "gemv-dot4", 4: "gemv-mfma"}[path]
    M, N = x_i8.shape[0], code.shape[0]
    announce(f"ternary_linear_acc {label} path={pname} M={M} N={N} K={x_i8.shape[1]}")
    acc = gpu_linear(twl, x_i8, a_scale, packed, q, smax, path, True)
    oacc = O.linear_acc(x_i8, code, oq)
    bad = np.argwhere(acc != oacc)
    assert bad.size == 0, f"{label}/{pname}: {len(bad)} acc mismatches, first {bad[:5].tolist()}"
    announce(f"ternary_linear {label} path={pname}")
    y = gpu_linear(twl, x_i8, a_scale, packed, q, smax, path, False)
    np.testing.assert_allclose(y, O.epilogue(oacc, a_scale, osm), rtol=Y_RTOL, atol=0)
    return acc, y


# ----------------------------------------------------------- the five configs

@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_rotate_quant_act_configs(twl, name):
    layer = W.make_config(name)
    _check_rotq(twl, layer.x_bits, layer.sign, name)


def test_config_tiny_end_to_end_both_paths(twl):
    layer = W.make_config("tiny")
    x_i8, a_scale = _check_rotq(twl, layer.x_bits, layer.sign, "tiny")
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "tiny")
    acc_gemm, _ = _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, 1, "tiny")
    acc_gemv, _ = _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, 2, "tiny")
    assert np.array_equal(acc_gemm, acc_gemv)
    # sanity against the unquantised float64 product ([P1] section 4: ~9.5e-3)
    y = gpu_linear(twl, x_i8, a_scale, packed, q, smax, 0, False)
    e = O.rel_err(y, O.float_reference(layer.x_bits, layer.sign, layer.code, layer.s_bits))
    assert 3e-3 < e < 2.5e-2, e


@pytest.mark.parametrize("name", ["prefill_gate_up", "prefill_down"])
def test_prefill_configs_full(twl, name):
    layer = W.make_config(name)
    x_i8, a_scale = _check_rotq(twl, layer.x_bits, layer.sign, name)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, name)
    _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, 0, name)


@pytest.mark.parametrize("name", ["decode_gate_up", "decode_down"])
def test_decode_sweep_full(twl, name):
    layer = W.make_config(name)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, name)
    for M in W.DECODE_MS:
        xb = np.ascontiguousarray(layer.x_bits[:M])
        x_i8, a_scale = _check_rotq(twl, xb, layer.sign, f"{name} M={M}")
        acc, _ = _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, 0,
                               f"{name} M={M}")
        # both decode kernels, whichever the automatic choice was
        for path in (twl.PATH_GEMV_DOT4, twl.PATH_GEMV_MFMA):
            announce(f"ternary_linear_acc {name} M={M} path={path}")
            assert np.array_equal(gpu_linear(twl, x_i8, a_scale, packed, q, smax, path, True), acc)


def test_stack_sampled_layers(twl):
    """64-layer stack: three layers spread over the stack, each of the three
    linears, prefill M=512 and decode M=24, inputs drawn on the GPU; the oracle
    checks rotation/quantisation in full and the linear on sampled outputs."""
    signs = W.stack_signs()
    rng = np.random.default_rng(99)
    for layer in (0, 37, 63):
        for which in range(3):
            name, K, N, _, _ = W.STACK_LINEARS[which]
            x_bits_d, code_d, s_bits_d = W.stack_linear_torch(layer, which, 512, "cuda")
            code_h = host(code_d)
            s_h = host(s_bits_d).view(np.uint16)
            lbl0 = f"stack L{layer} {name}"
            announce(f"pack_ternary {lbl0} N={N} K={K}")
            packed, q, smax = twl.pack_ternary(code_d, s_bits_d)
            oq, osm = O.decompose_scales(s_h)
            assert np.array_equal(host(q), oq), lbl0
            assert np.array_equal(host(smax).view(np.uint32), osm.view(np.uint32)), lbl0
            prow = rng.integers(0, N, 64)
            assert np.array_equal(O.untile_rows(host(packed), N, K)[prow],
                                  O.pack_rows(code_h[prow])), lbl0
            xb = host(x_bits_d).view(np.uint16)
            for M in (512, 24):
                lbl = f"stack L{layer} {name} M={M}"
                x_i8, a_scale = _check_rotq(twl, np.ascontiguousarray(xb[:M]), signs[K], lbl)
                announce(f"ternary_linear {lbl}")
                acc = gpu_linear(twl, x_i8, a_scale, packed, q, smax, 0, True)
                y = gpu_linear(twl, x_i8, a_scale, packed, q, smax, 0, False)
                rows = rng.integers(0, M, 256)
                cols = rng.integers(0, N, 256)
                oacc = O.linear_acc_at(x_i8, code_h, oq, rows, cols)
                assert np.array_equal(acc[rows, cols], oacc), lbl
                np.testing.assert_allclose(y[rows, cols], O.epilogue_at(oacc, a_scale, osm, rows, cols),
                                           rtol=Y_RTOL, atol=0)
            del code_d, code_h


# ------------------------------------------------ tiles, ragged tails, edges

@pytest.mark.parametrize("M,N,K", [(300, 200, 2048), (25, 513, 1024), (64, 64, 1024),
                                   (257, 257, 3072), (512, 1024, 1024), (129, 96, 4096)])
def test_gemm_ragged_shapes(twl, M, N, K):
    layer = W.make_layer(1000 + M + N, M, K, N, codes="sparse40")
    x_i8, a_scale = _check_rotq(twl, layer.x_bits, layer.sign, "ragged")
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "ragged")
    _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, 1, f"ragged {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [
    (511, 17408, 1024),   # last row tile one row short
    (449, 34816, 2048),   # last row tile of 65 rows; two rounds of workgroups
    (1000, 24580, 1024),  # ragged rows and columns (N % 8 == 4)
    (1000, 8704, 1024)])
def test_gemm_12_wave_tile_ragged(twl, M, N, K):
    # the 128 x 288 tile of 12 waves (the prefill gate/up plan) with M and N
    # not multiples of the tile, as the planner picks it for these shapes
    plan = twl.plan_info(M, N, K)
    assert (plan["family"], plan["tile_rows"], plan["tile_cols"], plan["waves"], plan["splits"]) == \
        ("gemm", 128, 288, 12, 1), plan
    layer = W.make_layer(9000 + M + N, M, K, N)
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "12-wave ragged")
    _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, twl.PATH_AUTO,
                  f"12-wave ragged {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 17, 24])
@pytest.mark.parametrize("N,K", [(1, 1024), (65, 2048), (1000, 5120),
                                 # row-balanced decode: 40-41 rows per workgroup,
                                 # 95-96 rows, and two rounds of workgroups (48 rows)
                                 (10241, 2048), (24575, 1024), (24577, 1024),
                                 # one 32-row subtile: 16-17 rows per workgroup with
                                 # 3 groups per wave, 31-32 rows with 9 groups per wave
                                 (4100, 3072), (8000, 9216),
                                 # up to 16 tokens, 16-row subtiles: 16 rows per
                                 # workgroup (one subtile), 62-63 rows (four)
                                 (4096, 2048), (16000, 1024),
                                 # five rounds of workgroups, 78-79 rows each
                                 (100003, 1024)])
def test_gemv_vs_gemm_shapes(twl, M, N, K):
    # every decode kernel (automatic choice, dot4, MFMA) and the GEMM against
    # the oracle, bit-exact in acc
    _gemv_vs_gemm(twl, M, N, K)


@pytest.mark.parametrize("M", [1, 16, 17, 20, 24])
@pytest.mark.parametrize("N,K", [
    # 5-group waves (K = 5120), each depth of loads in flight the planner
    # picks: 20 and 16 rows per workgroup (all five at M <= 16), 67-68 rows
    # in 16-row subtiles (three, issued early), two rounds of workgroups (two);
    # above 16 tokens one group, issued early, on every shape: 32-row
    # subtiles where 16-row ones pad no less (16, 20, 96 rows), else 16-row
    # subtiles with two 16-token operands (67-68 rows, 46-47 rows, and 68-69
    # rows in two rounds of workgroups; M = 17 and 20 leave the second
    # operand nearly empty);
    # 17-group waves (K = 17408) with 16-row subtiles (three, early); waves
    # with fewer groups than their bound (4 of 5 at K = 4096, 16 of 17 at
    # K = 16384), where the last groups' loads are clamped re-reads
    (5120, 5120), (4096, 5120), (17407, 5120), (24577, 5120), (34817, 5120), (6000, 17408),
    (12000, 4096), (5120, 16384)])
def test_gemv_prefetch_depths(twl, M, N, K):
    _gemv_vs_gemm(twl, M, N, K)


def _gemv_vs_gemm(twl, M, N, K):
    layer = W.make_layer(2000 + M * 7 + N, M, K, N)
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "gemv")
    accs = []
    for path, name in ((twl.PATH_GEMV, "gemv"), (twl.PATH_GEMV_DOT4, "dot4"),
                       (twl.PATH_GEMV_MFMA, "decode-mfma"), (twl.PATH_GEMM, "gemm")):
        a, _ = _check_linear(twl, x_i8, a_scale, packed, q, smax, layer.code, oq, osm, path,
                             f"{name} M={M}")
        accs.append(a)
    for a in accs[1:]:
        assert np.array_equal(accs[0], a)


@pytest.mark.parametrize("path", ["dot4", "mfma"])
@pytest.mark.parametrize("M,N,K", [(1, 129, 32768), (5, 64, 65536), (24, 200, 20480)])
def test_gemv_k_split_across_workgroups(twl, M, N, K, path):
    # K large enough that the GEMV splits it over several workgroups per row
    # block (partial sums in the workspace, added by a second kernel).
    # Repeated calls on one workspace, interleaved with a GEMM call on it,
    # must give identical results.
    dpath = twl.PATH_GEMV_DOT4 if path == "dot4" else twl.PATH_GEMV_MFMA
    layer = W.make_layer(3000 + M + N, M, K, N, codes="sparse40")
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "k-split")
    oacc = O.linear_acc(x_i8, layer.code, oq)
    oy = O.epilogue(oacc, a_scale, osm)
    xi, sc = dev(x_i8), dev(a_scale)
    ws = torch.full((max(1, twl.workspace_bytes(M, N, K)),), 0x5A, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        announce(f"{path} k-split M={M} N={N} K={K} rep={rep}")
        acc = host(twl.ternary_linear_acc(xi, packed, q, path=dpath, workspace=ws))
        assert np.array_equal(acc, oacc), f"rep {rep}: acc differs"
        y = host(twl.ternary_linear(xi, sc, packed, q, smax, path=dpath, workspace=ws))
        np.testing.assert_allclose(y, oy, rtol=Y_RTOL, atol=0)
        announce(f"gemm on the same workspace M={M} N={N} K={K} rep={rep}")
        acc2 = host(twl.ternary_linear_acc(xi, packed, q, path=twl.PATH_GEMM, workspace=ws))
        assert np.array_equal(acc2, oacc), f"rep {rep}: GEMM acc differs"


def _extreme_operands(M, N, K, seed):
    """x_i8 rows of +127, -127 or random; code rows of +1, -1 or random; all
    scales equal, so q = 127 everywhere and acc reaches +-127*127*K."""
    rng = np.random.default_rng(seed)
    x_i8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    x_i8[0::3] = 127
    x_i8[1::3] = -127
    code = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    code[0::3] = 1
    code[1::3] = -1
    s_bits = np.full((N, K // 128), 0.02, dtype=np.float16).view(np.uint16)
    a_scale = rng.uniform(0.5, 2.0, M).astype(np.float32)
    return x_i8, a_scale, code, s_bits


@pytest.mark.parametrize("M,N,K,paths", [
    # the GEMM at the largest K the library takes (split over K)
    (300, 130, 65536, ("gemm",)),
    # the dot4 and K-split matrix-core decode kernels at the largest K
    (1, 130, 65536, ("dot4", "mfma")),
    (24, 130, 65536, ("dot4", "mfma")),
    # the row-balanced decode kernel (>= 16 rows per CU) at its largest K:
    # 8 waves x 33 groups of 128
    (24, 4096, 33792, ("gemv", "gemm")),
])
def test_extreme_accumulators_at_max_k(twl, M, N, K, paths):
    x_i8, a_scale, code, s_bits = _extreme_operands(M, N, K, 4000 + M + N)
    packed, q, smax, oq, osm = _check_pack(twl, code, s_bits, f"extreme K={K}")
    assert (oq == 127).all()
    oacc = O.linear_acc(x_i8, code, oq)
    # the oracle itself at the closed form: +-127*127*K where both rows are
    # constant (same sign -> +, opposite -> -)
    big = 127 * 127 * K
    assert big < 2 ** 31
    assert (oacc[0::3, 0::3] == big).all() and (oacc[1::3, 1::3] == big).all()
    assert (oacc[0::3, 1::3] == -big).all() and (oacc[1::3, 0::3] == -big).all()
    ids = {"gemm": twl.PATH_GEMM, "gemv": twl.PATH_GEMV, "dot4": twl.PATH_GEMV_DOT4,
           "mfma": twl.PATH_GEMV_MFMA}
    for name in paths:
        _check_linear(twl, x_i8, a_scale, packed, q, smax, code, oq, osm, ids[name],
                      f"extreme {name} M={M}")


@pytest.mark.parametrize("N", [5536, 5534])
def test_gemm_split_k_with_padding_fragments(twl, N):
    # a 128 x 288 tile (nine column fragments over two column waves, so one
    # wave role holds a padding fragment) with three splits: the split-K
    # reduce skips the padding fragment and stores the ragged last tile
    # (N = 5536: 16-byte stores; N = 5534: element stores)
    M, K = 512, 17408
    rng = np.random.default_rng(5000 + N)
    x_i8 = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    a_scale = rng.uniform(0.01, 0.1, M).astype(np.float32)
    code = rng.choice(np.array([-1, 0, 1], dtype=np.int8), size=(N, K), p=[0.3, 0.4, 0.3])
    s_bits = np.exp(rng.normal(-4, 0.5, (N, K // 128))).astype(np.float16).view(np.uint16)
    packed, q, smax, oq, osm = _check_pack(twl, code, s_bits, f"split-K padding N={N}")
    _check_linear(twl, x_i8, a_scale, packed, q, smax, code, oq, osm, twl.PATH_GEMM,
                  f"split-K padding {M}x{N}x{K}")


def test_rotate_edge_cases(twl):
    # maximum width (64 blocks), one token
    layer = W.make_layer(31, 2, 65536, 1)
    _check_rotq(twl, layer.x_bits, layer.sign, "K=65536")
    # a zero token and a single-spike token
    x = np.zeros((3, 2048), dtype=np.uint16)
    x[1, 7] = W.f32_to_bf16_bits(np.array([3.0], dtype=np.float32))[0]
    x[2] = W.f32_to_bf16_bits(np.linspace(-4, 4, 2048, dtype=np.float32))
    sign = np.where(np.arange(2048) % 3 == 0, -1, 1).astype(np.int8)
    gx, gs = _check_rotq(twl, x, sign, "zero/spike")
    assert gs[0] == 0 and not gx[0].any()
    # 17 blocks (odd count, two blocks per wave)
    layer = W.make_layer(32, 5, 17408, 1, act="silu_gate")
    _check_rotq(twl, layer.x_bits, layer.sign, "K=17408")


def test_pack_edge_cases(twl):
    # an all-zero scale row, a negative scale, and invalid codes
    code = np.random.default_rng(3).integers(-1, 2, size=(4, 1024)).astype(np.int8)
    s = np.full((4, 8), 0.01, dtype=np.float16)
    s[1] = 0
    s[2, 3] = -0.02
    _check_pack(twl, code, s.view(np.uint16), "zero/negative scales")
    bad_code = code.copy()
    bad_code[3, 5] = 2
    bad_code[3, 900] = -7
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    packed, _, _ = gpu_pack(twl, bad_code, s.view(np.uint16), bad=counter)
    assert int(host(counter)[0]) == 2
    fixed = bad_code.copy()
    fixed[3, 5] = 0
    fixed[3, 900] = 0
    assert np.array_equal(host(packed).reshape(-1), O.pack_codes(fixed).reshape(-1))


def test_empty_inputs(twl):
    x = torch.empty((0, 1024), dtype=torch.int16, device="cuda")
    sign = torch.ones(1024, dtype=torch.int8, device="cuda")
    xi, sc = twl.rotate_quant_act(x, sign)
    assert xi.shape == (0, 1024)
    layer = W.make_layer(5, 1, 1024, 8)
    packed, q, smax = gpu_pack(twl, layer.code, layer.s_bits)
    y = twl.ternary_linear(torch.empty((0, 1024), dtype=torch.int8, device="cuda"),
                           torch.empty(0, device="cuda"), packed, q, smax)
    assert y.shape == (0, 8)


def test_shape_errors_enqueue_nothing(twl):
    x = torch.zeros((4, 1000), dtype=torch.int16, device="cuda")
    sign = torch.ones(1000, dtype=torch.int8, device="cuda")
    with pytest.raises(twl.TwlError) as e:
        twl.rotate_quant_act(x, sign)
    assert e.value.status == 2


def test_repeat_runs_are_bitwise_identical(twl):
    layer = W.make_config("prefill_down")
    x = dev(layer.x_bits.view(np.int16))
    sign = dev(layer.sign)
    packed, q, smax = gpu_pack(twl, layer.code, layer.s_bits)
    outs = []
    for _ in range(2):
        announce("repeat prefill_down")
        xi, sc = twl.rotate_quant_act(x, sign)
        outs.append((host(xi), host(twl.ternary_linear(xi, sc, packed, q, smax))))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


# ------------------------------------------------- bf16 output option (R12)

@pytest.mark.parametrize("M,N,K,path", [
    (300, 513, 2048, "gemm"),            # ragged GEMM tiles, N odd: scalar stores
    (257, 1024, 3072, "gemm"),           # N % 8 == 0: 16-byte bf16 stores, ragged M
    (40, 300, 32768, "gemm"),            # GEMM with split-K partials, N % 8 == 4
    (3, 1000, 5120, "gemv_dot4"),        # dot4 decode
    (9, 200, 20480, "gemv_mfma"),        # MFMA decode, K split over workgroups
    (17, 24575, 1024, "gemv_mfma"),      # MFMA decode, row-balanced
])
def test_bf16_output(twl, M, N, K, path):
    # y in bf16 is the fp32 y rounded to nearest even in the epilogue: equal
    # bit for bit to rounding the kernel's own fp32 y, and within half a bf16
    # ulp (2^-8 relative) of the oracle's y
    p = {"gemm": twl.PATH_GEMM, "gemv_dot4": twl.PATH_GEMV_DOT4, "gemv_mfma": twl.PATH_GEMV_MFMA}[path]
    layer = W.make_layer(4000 + M + N, M, K, N, codes="sparse40")
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, "bf16")
    oy = O.epilogue(O.linear_acc(x_i8, layer.code, oq), a_scale, osm)
    xi, sc = dev(x_i8), dev(a_scale)
    announce(f"ternary_linear fp32 and bf16 {path} M={M} N={N} K={K}")
    y32 = host(twl.ternary_linear(xi, sc, packed, q, smax, path=p))
    y16 = host(twl.ternary_linear_bf16(xi, sc, packed, q, smax, path=p).view(torch.int16)).view(np.uint16)
    np.testing.assert_allclose(y32, oy, rtol=Y_RTOL, atol=0)
    assert np.array_equal(y16, O.round_bf16(y32))
    y16f = (y16.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(y16f.astype(np.float64) - oy) <= 2.0**-8 * np.abs(oy.astype(np.float64)))


@pytest.mark.parametrize("name,M,N,K,path,store", [
    # prefill gate/up in full: the GEMM's own epilogue (no split-K), N % 8 == 0:
    # 16-byte bf16 stores
    ("prefill_gate_up", 512, 17408, 5120, "auto", "bf16x8"),
    # N % 8 == 4: 8-byte bf16 stores of four columns
    ("ragged_n8", 300, 24580, 1024, "gemm", "bf16x4"),
    # N % 4 != 0: element stores straight from the accumulators
    ("ragged_n4", 24, 24577, 1024, "gemm", "element"),
])
def test_bf16_output_gemm_epilogue_without_split(twl, name, M, N, K, path, store):
    # bf16 y written by the GEMM's own store path (not the split-K reduce):
    # the plan must not split K, so the tile's epilogue rounds and stores
    p = {"auto": twl.PATH_AUTO, "gemm": twl.PATH_GEMM}[path]
    plan = twl.plan_info(M, N, K, p)
    assert plan["family"] == "gemm" and plan["splits"] == 1 and plan["reduce_kernel"] == 0, plan
    if name == "prefill_gate_up":
        layer = W.make_config(name)
    else:
        layer = W.make_layer(8000 + M + N, M, K, N, codes="sparse40")
    x_i8, a_scale = O.rotate_quant_act(layer.x_bits, layer.sign)
    packed, q, smax, oq, osm = _check_pack(twl, layer.code, layer.s_bits, f"bf16 {name}")
    oy = O.epilogue(O.linear_acc(x_i8, layer.code, oq), a_scale, osm)
    xi, sc = dev(x_i8), dev(a_scale)
    announce(f"ternary_linear fp32 and bf16 {name} ({store}) M={M} N={N} K={K} plan={plan}")
    y32 = host(twl.ternary_linear(xi, sc, packed, q, smax, path=p))
    y16 = host(twl.ternary_linear_bf16(xi, sc, packed, q, smax, path=p).view(torch.int16)).view(np.uint16)
    np.testing.assert_allclose(y32, oy, rtol=Y_RTOL, atol=0)
    assert np.array_equal(y16, O.round_bf16(y32))
    y16f = (y16.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(y16f.astype(np.float64) - oy) <= 2.0**-8 * np.abs(oy.astype(np.float64)))


# ------------------------------- fused SiLU(gate) * up rotation (R13, R14)

@pytest.mark.parametrize("M,K", [(256, 17408), (1, 17408), (24, 17408), (7, 5120), (3, 65536)])
def test_silu_mul_rotate_quant_act(twl, M, K):
    gu, sign = W.make_gate_up(5000 + M + K, M, K)
    announce(f"silu_mul_rotate_quant_act M={M} K={K}")
    xi, sc = twl.silu_mul_rotate_quant_act(dev(gu.view(np.int16)), dev(sign))
    ox, osc = O.silu_mul_rotate_quant_act(gu, sign)
    assert np.array_equal(host(sc).view(np.uint32), osc.view(np.uint32))
    bad = np.argwhere(host(xi) != ox)
    assert bad.size == 0, f"{len(bad)} x_i8 mismatches, first {bad[:5].tolist()}"


def test_silu_mul_rotate_edge_values(twl):
    # the clamp of exp's argument (|gate| > 87), zeros, and tokens whose
    # activation is all zero (a_scale = 0)
    K = 2048
    g = np.zeros((4, K), dtype=np.float32)
    u = np.ones((4, K), dtype=np.float32)
    g[0] = np.linspace(-300, 300, K)
    g[1] = -120.0
    u[1] = 1e30
    g[2] = 0.0                      # SiLU(0) = 0: zero token
    g[3] = np.linspace(-4, 4, K)
    u[3, ::2] = 0.0
    gu = np.concatenate([W.f32_to_bf16_bits(g), W.f32_to_bf16_bits(u)], axis=1)
    sign = np.where(np.arange(K) % 5 == 0, -1, 1).astype(np.int8)
    announce("silu_mul_rotate_quant_act edge values")
    xi, sc = twl.silu_mul_rotate_quant_act(dev(gu.view(np.int16)), dev(sign))
    ox, osc = O.silu_mul_rotate_quant_act(gu, sign)
    assert np.array_equal(host(sc).view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(host(xi), ox)
    assert osc[2] == 0


# ------------------------------------------- bf16 reference path (R15)

@pytest.mark.parametrize("M,N,K,rows", [(16, 256, 1024, None), (300, 513, 2048, None),
                                        (1, 17408, 5120, None), (512, 17408, 5120, 48)])
def test_reference_linear_bf16(twl, M, N, K, rows):
    # the rotation alone is bit-exact; y within the fp32 accumulation bound of
    # the exact sum (rows: check a sample of token rows of a large layer)
    layer = W.make_layer(6000 + M + N, M, K, N)
    announce(f"rotate_act_bf16 M={M} K={K}")
    r = twl.rotate_act_bf16(dev(layer.x_bits.view(np.int16)), dev(layer.sign))
    r_bits = host(r.view(torch.int16)).view(np.uint16)
    assert np.array_equal(r_bits, O.rotate_bf16(layer.x_bits, layer.sign))
    packed, _, _ = twl.pack_ternary(dev(layer.code), dev(layer.s_bits.view(np.int16)))
    announce(f"reference_linear_bf16 M={M} N={N} K={K}")
    y = host(twl.reference_linear_bf16(r, packed, dev(layer.s_bits.view(np.int16))))
    sel = np.arange(M) if rows is None else np.random.default_rng(1).choice(M, rows, replace=False)
    want, scale = O.reference_linear_bf16(r_bits[sel], layer.code, layer.s_bits)
    err = np.abs(y[sel].astype(np.float64) - want)
    assert np.all(err <= K * 2.0**-24 * scale + 1e-30), float(np.max(err / (scale + 1e-30)))


# ------------------------------------------------------ HIP graph replays

@pytest.mark.parametrize("M,N,K", [(512, 1000, 5120),    # GEMM
                                   (512, 17408, 1024),   # GEMM, 12-wave 128x288 tiles
                                   (40, 300, 32768),     # GEMM with split-K partials
                                   (9, 200, 20480),      # MFMA decode, K slices + reduce
                                   (5, 24575, 1024),     # row-balanced MFMA decode
                                   (1, 5120, 17408),     # row-balanced, one subtile, 17 groups/wave
                                   (24, 17408, 5120),    # row-balanced, three subtiles, 24 tokens
                                   (2, 1000, 5120)])     # dot4 decode
def test_graph_replays_match_eager(twl, M, N, K):
    # the path (rotation + linear) captured once in a graph; every replay,
    # with eager work on the same buffers in between, must give the eager
    # result bit for bit (the library records no memset and allocates nothing)
    layer = W.make_layer(7000 + M + N, M, K, N)
    x, sign = dev(layer.x_bits.view(np.int16)), dev(layer.sign)
    packed, q, smax = twl.pack_ternary(dev(layer.code), dev(layer.s_bits.view(np.int16)))
    x_i8 = torch.empty((M, K), dtype=torch.int8, device="cuda")
    a_scale = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.full((max(1, twl.workspace_bytes(M, N, K)),), 0x5A, dtype=torch.uint8, device="cuda")

    def step():
        twl.rotate_quant_act(x, sign, out=(x_i8, a_scale))
        twl.ternary_linear(x_i8, a_scale, packed, q, smax, out=y, workspace=ws)

    announce(f"graph capture M={M} N={N} K={K}")
    step()
    want_y, want_x = host(y).copy(), host(x_i8).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step()
    for rep in range(4):
        y.fill_(float("nan"))
        x_i8.zero_()
        announce(f"graph replay {rep} M={M} N={N} K={K}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(x_i8), want_x), f"replay {rep}: x_i8"
        assert np.array_equal(host(y).view(np.uint32), want_y.view(np.uint32)), f"replay {rep}: y"
        # eager work on the same workspace between replays
        twl.ternary_linear_acc(x_i8, packed, q, workspace=ws)
        torch.cuda.synchronize()
    oy = O.ternary_linear(*O.rotate_quant_act(layer.x_bits, layer.sign), layer.code,
                          *O.decompose_scales(layer.s_bits))
    np.testing.assert_allclose(want_y, oy, rtol=Y_RTOL, atol=0)


# ------------------------------------------------------------ plan queries

@pytest.mark.parametrize("M,N,K,path,family", [
    (512, 17408, 5120, 0, "gemm"), (256, 5120, 17408, 0, "gemm"),
    (1, 17408, 5120, 0, "decode_rows"), (24, 5120, 17408, 0, "decode_rows"),
    (2, 1000, 5120, 0, "decode_dot4"), (9, 200, 20480, 0, "decode_mfma"),
    (24, 5120, 17408, 3, "decode_dot4"), (24, 5120, 17408, 1, "gemm")])
def test_plan_info_matches_workspace_and_family(twl, M, N, K, path, family):
    plan = twl.plan_info(M, N, K, path)
    assert plan["family"] == family, plan
    assert plan["splits"] >= 1 and plan["workgroups"] >= 1 and plan["waves"] >= 1
    assert plan["reduce_kernel"] == (1 if plan["splits"] > 1 else 0)
    assert plan["workspace_bytes"] <= twl.workspace_bytes(M, N, K)
    assert (plan["workspace_bytes"] > 0) == (plan["splits"] > 1)


# ------------- rotate_quant_linear: the layer from bf16 x, fused at small M

@pytest.mark.parametrize("M,N,K,silu,fused", [
    (1, 17408, 5120, False, True),   # decode gate/up: 5 blocks over 8 waves
    (2, 17408, 5120, True, True),    # the SiLU form, 10 blocks
    (2, 16001, 2048, False, True),   # ragged rows (62-63 per workgroup), 4 blocks
    (1, 5120, 5120, False, True),    # 20 rows per workgroup: two subtiles, loads issued early
    (2, 5120, 5120, True, True),
    (1, 5120, 17408, True, True),    # decode down with its SiLU input: 17 blocks
    (1, 5120, 17408, False, True),
    (1, 8000, 9216, True, True),     # 31-32 rows per workgroup, 9 groups per wave
    (3, 24577, 2048, False, False),  # three tokens: two steps
    (4, 17408, 5120, False, False),
    (2, 24577, 1024, False, False),  # two rounds of workgroups: two steps
    (1, 34816, 5120, False, False),
    (2, 5120, 17408, False, False),  # 34 blocks: more than 2 per wave, two steps
    (5, 17408, 5120, False, False),
    (64, 2048, 2048, True, False),   # prefill: the GEMM path
])
def test_rotate_quant_linear(twl, M, N, K, silu, fused):
    layer = W.make_layer(7000 + M + N + K, M, K, N)
    if silu:
        xin, sign = W.make_gate_up(7100 + M + K, M, K)
        ox, osc = O.silu_mul_rotate_quant_act(xin, sign)
    else:
        xin, sign = layer.x_bits.copy(), layer.sign
        if M >= 2:
            xin[1] = 0  # an all-zero token: a_scale 0, x_i8 0
        ox, osc = O.rotate_quant_act(xin, sign)
    packed, q, smax = gpu_pack(twl, layer.code, layer.s_bits)
    oq, osm = O.decompose_scales(layer.s_bits)
    assert twl.rotate_quant_linear_fused(M, N, K) == fused
    announce(f"rotate_quant_linear M={M} N={N} K={K} silu={silu} fused={fused}")
    x, sg = dev(xin.view(np.int16)), dev(sign)
    y, xi, sc = twl.rotate_quant_linear(x, sg, packed, q, smax, silu=silu)
    acc = twl.rotate_quant_linear(x, sg, packed, q, smax, silu=silu, out_dtype=torch.int32)[0]
    yb = twl.rotate_quant_linear(x, sg, packed, q, smax, silu=silu, out_dtype=torch.bfloat16)[0]
    assert np.array_equal(host(sc).view(np.uint32), osc.view(np.uint32)), "a_scale differs"
    bad = np.argwhere(host(xi) != ox)
    assert bad.size == 0, f"{len(bad)} x_i8 mismatches, first {bad[:5].tolist()}"
    oacc = O.linear_acc(ox, layer.code, oq)
    bad = np.argwhere(host(acc) != oacc)
    assert bad.size == 0, f"{len(bad)} acc mismatches, first {bad[:5].tolist()}"
    np.testing.assert_allclose(host(y), O.epilogue(oacc, osc, osm), rtol=Y_RTOL, atol=0)
    # bit for bit what the two calls give
    rot = twl.silu_mul_rotate_quant_act if silu else twl.rotate_quant_act
    xi2, sc2 = rot(x, sg)
    assert torch.equal(y, twl.ternary_linear(xi2, sc2, packed, q, smax))
    assert torch.equal(yb, twl.ternary_linear_bf16(xi2, sc2, packed, q, smax))


def test_rotate_quant_linear_graph_replays(twl):
    # the fused kernel captured in a HIP graph: every replay equals the eager call
    M, N, K = 2, 17408, 5120
    layer = W.make_layer(7300, M, K, N)
    packed, q, smax = gpu_pack(twl, layer.code, layer.s_bits)
    assert twl.rotate_quant_linear_fused(M, N, K)
    x, sg = dev(layer.x_bits.view(np.int16)), dev(layer.sign)
    announce("rotate_quant_linear graph replays")
    y0 = twl.rotate_quant_linear(x, sg, packed, q, smax)[0].clone()
    y = torch.empty_like(y0)
    xi = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sc = torch.empty((M,), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        twl.rotate_quant_linear(x, sg, packed, q, smax, out=y, x_i8=xi, a_scale=sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        twl.rotate_quant_linear(x, sg, packed, q, smax, out=y, x_i8=xi, a_scale=sc)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
