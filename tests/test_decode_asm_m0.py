"""The decode kernels' direct global->LDS loads set m0 inside their own inline
assembly, which cannot declare m0 clobbered. That is only sound while the
compiler itself neither reads nor writes m0 anywhere in those kernels: this
test builds the kernels' gfx950 assembly with the library's flags and checks
that every instruction naming m0 sits inside an inline-assembly block."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_moe_transformer_amd import build as B

SRC = os.path.join(B.CSRC, "moe_gemm_decode.hip")


def _device_asm(tmp_path) -> str:
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "decode.s"
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def m0_outside_inline_asm(asm: str):
    """(function, line, instruction) of every instruction naming m0 that is
    not between ;;#ASMSTART and ;;#ASMEND, and the count of those inside."""
    inside, fn, outside, n_inside = False, None, [], 0
    for i, line in enumerate(asm.split("\n")):
        if re.match(r"^_Z\S+:$", line):
            fn = line[:-1]
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0]
        if re.search(r"\bm0\b", code):
            if inside:
                n_inside += 1
            else:
                outside.append((fn, i + 1, code.strip()))
    return outside, n_inside


def test_scanner_finds_a_compiler_use_of_m0():
    asm = "\n".join(["_Zk:", "\t;;#ASMSTART", "\ts_mov_b32 m0, s3", "\t;;#ASMEND",
                     "\ts_mov_b32 m0, s4", "\tds_read_b32 v0, v1"])
    outside, n_inside = m0_outside_inline_asm(asm)
    assert n_inside == 1 and [o[2] for o in outside] == ["s_mov_b32 m0, s4"]


def test_decode_kernels_leave_m0_to_their_inline_asm(tmp_path):
    outside, n_inside = m0_outside_inline_asm(_device_asm(tmp_path))
    assert n_inside > 0, "no direct loads found in the decode kernels' assembly"
    assert outside == [], f"compiler-generated uses of m0: {outside[:5]}"
