"""The library's device code holds no packed-FP32 instructions.

The build passes `-Xclang -target-feature -Xclang -packed-fp32-ops` so that
hipcc never forms v_pk_add_f32, v_pk_mul_f32 or v_pk_fma_f32 from ordinary
float code (some forms of them have given wrong results on these GPUs).  The
host pass warns that it does not know the feature; the device pass applies it.
This test compiles every source to gfx950 assembly with the build's own flags
and checks the mnemonics, and checks once without the flag that the compiler
would otherwise form them (so the check can fail).  CPU only: hipcc
cross-compiles.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from w4a16_routed_experts_amd import build

PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
FLAG = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _device_asm(src: str, tmp_path, with_flag: bool = True) -> str:
    cmd = build.build_command(str(tmp_path / "unused.so"))
    # the build's compiler and flags, for device code only, to assembly
    cmd = [c for c in cmd if c not in ("-shared",) and not c.endswith(".hip")]
    i = cmd.index("-o")
    del cmd[i:i + 2]
    if not with_flag:
        for j in range(len(cmd) - len(FLAG) + 1):
            if cmd[j:j + len(FLAG)] == FLAG:
                del cmd[j:j + len(FLAG)]
                break
    out = tmp_path / (os.path.basename(src) + (".s" if with_flag else ".noflag.s"))
    res = subprocess.run(cmd + ["--cuda-device-only", "-S", "-o", str(out), os.path.join(build.CSRC, src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


needs_hipcc = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                 reason="hipcc is not installed")


@needs_hipcc
@pytest.mark.parametrize("src", build.SOURCES)
def test_no_packed_fp32_in_device_code(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    hits = sorted({m.group(0) for m in PACKED_F32.finditer(asm)})
    assert not hits, f"{src}: {hits}"


@needs_hipcc
def test_check_bites_without_the_flag(tmp_path):
    asm = _device_asm("decode.hip", tmp_path, with_flag=False)
    assert PACKED_F32.search(asm), "without the flag the compiler forms packed-FP32 instructions here"
