"""Checks on the generated gfx950 code that need no GPU.

The GEMM and the row-balanced decode kernel issue their direct global->LDS
loads from inline asm that sets M0 itself.  LLVM treats M0 as a reserved
register and does not preserve it around inline asm, so these kernels are only
correct while the compiler never uses M0 for anything else.  This test
compiles both sources to assembly with the library's own flags and checks, in
every instantiation of those kernels, that every M0 write is one of ours (an
s_mov_b32 from an SGPR followed by a global_load_lds) and that M0 is read by
nothing else.  It also checks the GEMM's main loop keeps a single vmcnt wait
per pipeline stage and no accumulator copies.
"""
import os
import re
import shutil
import subprocess

import pytest

from ternary_weight_linear_block_amd import build as B

# source file -> (kernel whose instantiations set M0 from inline asm, the
# least number of instantiations expected)
M0_KERNELS = {"gemm_i8.hip": ("gemm_kernel", 10),
              "gemv.hip": ("gemv_rows_kernel", 15)}


def _compile_asm(tmp_path_factory, src):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (os.path.splitext(src)[0] + ".s")
    cmd = [B.hipcc()] + [f for f in B.COMMON_FLAGS if f != "-fPIC"] + [
        "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile_asm(tmp_path_factory, "gemm_i8.hip")


def _kernels(asm_text, kernel="gemm_kernel", least=10):
    """name -> body for each instantiation of `kernel`."""
    out = {}
    for m in re.finditer(r"^(_Z\S*" + kernel + r"I\S*):[^\n]*\n(.*?)^\.Lfunc_end", asm_text, re.S | re.M):
        out[m.group(1)] = m.group(2)
    assert len(out) >= least, f"expected every {kernel} instantiation, found {len(out)}"
    return out


@pytest.mark.parametrize("src", sorted(M0_KERNELS))
def test_m0_only_feeds_our_lds_loads(tmp_path_factory, asm, src):
    text = asm if src == "gemm_i8.hip" else _compile_asm(tmp_path_factory, src)
    kernel, least = M0_KERNELS[src]
    kernels = _kernels(text, kernel, least)
    for name, body in kernels.items():
        lines = [ln.strip() for ln in body.splitlines() if ln.strip() and not ln.strip().startswith(";")]
        # gemv_rows_kernel<NS, GMAX, P, MAXT, ROT, RS, EARLY>: ROT is the fifth
        # template argument (the first bool)
        rot = re.search(r"gemv_rows_kernelI(?:Li\d+E){4}Lb([01])E", name)
        if src == "gemv.hip" and rot and rot.group(1) == "1":
            # the fused-rotation decode kernels quantise x into LDS themselves:
            # no direct loads, and so no M0 at all
            assert not any("global_load_lds" in ln or "m0" in ln for ln in lines), name
            continue
        assert "global_load_lds" in body, name
        for i, ln in enumerate(lines):
            if "m0" not in ln:
                continue
            if ln.startswith("s_mov_b32 m0, s"):
                nxt = lines[i + 1] if i + 1 < len(lines) else ""
                assert nxt.startswith("global_load_lds"), (name, ln, nxt)
            else:
                pytest.fail(f"{name}: compiler-generated use of m0: {ln}")


def _loops(body):
    """Innermost loops of a kernel body as text: the header block plus every
    block the compiler annotates as belonging to it (rotated loops put blocks
    before the header), each block running to the next label."""
    lines = body.splitlines()
    label_re = re.compile(r"^(\.LBB\w+|; %bb\.\d+):")
    blocks, cur = [], None
    for ln in lines:
        m = label_re.match(ln.strip())
        if m:
            cur = [ln]
            blocks.append(cur)
        elif cur is not None:
            cur.append(ln)
    loops = {}
    for b in blocks:
        head = b[0]
        m = re.search(r"Header=(BB\w+)", head)
        if "Inner Loop Header" in head:
            key = head.split(":")[0].strip()[2:]   # ".LBBn_m" -> "BBn_m"
        elif m:
            key = m.group(1)
        else:
            continue
        loops.setdefault(key, []).append("\n".join(b))
    return {k: "\n".join(v) for k, v in loops.items()}


def test_main_loop_has_one_wait_per_stage_and_no_accumulator_copies(asm):
    # the stage loop is unrolled by a whole number of pipeline stages: one
    # vmcnt wait per stage (RM x ceil(FN/WN) x 4/WK MFMAs), no AGPR copies
    for name, body in _kernels(asm).items():
        rm, fn, wk, wn = (int(v) for v in
                          re.search(r"gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name).groups())
        mains = [t for t in _loops(body).values() if "v_mfma" in t]
        assert len(mains) == 1, (name, len(mains))
        loop = mains[0]
        n_mfma = loop.count("v_mfma_i32_32x32x32_i8")
        per_stage = rm * ((fn + wn - 1) // wn) * (4 // wk)
        assert n_mfma > 0 and n_mfma % per_stage == 0, (name, n_mfma)
        assert loop.count("vmcnt") == n_mfma // per_stage, name
        assert "v_accvgpr" not in loop, name
