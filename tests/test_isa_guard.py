"""A guard on the generated code of the wide INT8 GEMM (CPU only: hipcc
cross-compiles for gfx950 here).

Its K loop counts copies in flight with fixed vmcnt values.  Once the last
copy of a tile is issued, the BF16 kernel loads its epilogue's scales and
bias (three loads in every lane) and the last slices' waits then allow
"copies + 3" operations in flight.  That is right only while those three
loads are issued before the first such wait; a compiler that moved them
past the waits would let the last copies be read before they land.  This
test compiles the kernel to assembly and checks the order."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _kernel_asm(tmp_path, name_re):
    from quantized_diffusion_amd import build as B
    out = tmp_path / "gemm_i8.s"
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-I", os.path.join(ROOT, "quantized_diffusion_amd", "csrc"),
           "--cuda-device-only", "-S", os.path.join(ROOT, "quantized_diffusion_amd", "csrc", "gemm_i8.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        pytest.fail(f"hipcc failed: {r.stderr[-2000:]}")
    lines = out.read_text().splitlines()
    start = next(i for i, l in enumerate(lines) if re.match(name_re, l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    return lines[start:end + 1]


def test_w12_epilogue_loads_precede_the_waits_that_count_them(tmp_path):
    from quantized_diffusion_amd import build as B
    if not os.path.exists(B.hipcc()):
        pytest.skip("no hipcc")
    body = _kernel_asm(tmp_path, r"^_ZN2qd12_GLOBAL__N_118gemm_i8_w12_kernelILi0E.*:")
    # the epilogue operand loads: the only plain (non-LDS) global loads of the
    # BF16 kernel after its K loop starts, two dwords and one BF16 half
    loads = [i for i, l in enumerate(body)
             if re.search(r"\bglobal_load_(dword|ushort)\b", l) and "lds" not in l]
    assert len(loads) >= 3, "epilogue operand loads not found"
    last3 = loads[-3:]
    # the last slices' waits: vmcnt = 5 g + 3 (five copies per slice and thread)
    waits = [i for i, l in enumerate(body)
             if (m := re.search(r"s_waitcnt vmcnt\((\d+)\)", l)) and int(m.group(1)) in (3, 8, 13, 18)]
    assert waits, "the drain's waits (vmcnt 3 / 8 / 13 / 18) not found"
    assert max(last3) < min(waits), \
        f"epilogue loads at asm lines {last3} are not all before the first counted wait at line {min(waits)}"
    # and they follow the steady K loop (its waits keep 10 copies in flight)
    steady = [i for i, l in enumerate(body) if "s_waitcnt vmcnt(10)" in l]
    assert steady and min(last3) > max(steady)
