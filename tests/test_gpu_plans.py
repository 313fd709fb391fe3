"""The decode planner's choices on the decode layers: subtile form, token
operands, loads in flight per wave and early issue, as the library reports
them in its plan log (TWL_LOG).  These choices change speed, not results, so
the parity tests cannot see them; this pins them on the 256-CU MI355X where
they were measured.
"""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def twl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ternary_weight_linear_block_amd as m
    m.library()  # raises if libtwl.so is missing: no fallback exists
    return m


# (M, N, K) -> the end of the plan line: "<rows>-row subtiles x<count>[ (two
# 16-token operands)], <groups> in flight[, early]"
PLANS = [
    # 5120 -> 17408: 68 rows per workgroup, 5 groups per wave
    (1, 17408, 5120, "16-row subtiles x5, 2 in flight, early"),
    (8, 17408, 5120, "16-row subtiles x5, 2 in flight, early"),
    (16, 17408, 5120, "16-row subtiles x5, 1 in flight, early"),
    (24, 17408, 5120, "16-row subtiles x5 (two 16-token operands), 1 in flight, early"),
    # 17408 -> 5120: 20 rows, 17 groups per wave
    (1, 5120, 17408, "16-row subtiles x2, 3 in flight, early"),
    (16, 5120, 17408, "16-row subtiles x2, 3 in flight, early"),
    (24, 5120, 17408, "32-row subtiles x1, 5 in flight"),
    # 5120 -> 5120: 20 rows, 5 groups per wave
    (1, 5120, 5120, "16-row subtiles x2, 3 in flight, early"),
    (24, 5120, 5120, "32-row subtiles x1, 1 in flight, early"),
    # 5120 -> 34816: two rounds of workgroups of 68 rows
    (1, 34816, 5120, "16-row subtiles x5, 2 in flight"),
    (16, 34816, 5120, "16-row subtiles x5, 1 in flight, early"),
    (24, 34816, 5120, "16-row subtiles x5 (two 16-token operands), 1 in flight, early"),
]


@pytest.mark.parametrize("M,N,K,form", PLANS)
def test_decode_plan(twl, capfd, monkeypatch, M, N, K, form):
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the plans are those of a 256-CU device")
    x_i8 = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    a_scale = torch.ones((M,), dtype=torch.float32, device="cuda")
    packed = torch.zeros((twl.packed_bytes(N, K),), dtype=torch.uint8, device="cuda")
    q = torch.zeros((N, K // 128), dtype=torch.int8, device="cuda")
    smax = torch.ones((N,), dtype=torch.float32, device="cuda")
    capfd.readouterr()
    monkeypatch.setenv("TWL_LOG", "1")
    y = twl.ternary_linear(x_i8, a_scale, packed, q, smax)
    torch.cuda.synchronize()
    monkeypatch.delenv("TWL_LOG")
    lines = [ln for ln in capfd.readouterr().err.splitlines() if ln.startswith("[twl] gemv-rows")]
    assert lines, "no row-kernel plan line"
    assert lines[-1].endswith(form), lines[-1]
    assert torch.count_nonzero(y).item() == 0
