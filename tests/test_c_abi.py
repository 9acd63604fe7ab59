"""The boundary from C: a C11 program that includes only include/dfp.h
compiles with gcc, links the in-tree libdfp.so, and its host-side calls agree
with the same entry points reached through the Python binding (CPU only)."""
import os
import shutil
import subprocess

import pytest

from patch_attention_cfg_amd import dfp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_links_and_agrees(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(dfp.LIB_PATH):
        pytest.skip("gcc or the built library is missing")
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(dfp.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", str(exe),
           "-L", libdir, "-l:" + os.path.basename(dfp.LIB_PATH), "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True,
                         timeout=60).stdout.split("\n")
    got = {line.split(" ", 1)[0]: line.split(" ", 1)[1] for line in out if " " in line}
    assert out[-2] == "ok"
    cx, ce = (float(v) for v in got["ddim"].split())
    assert (cx, ce) == dfp.ddim_coeffs(0.5, 0.75)
    cx, ce = (float(v) for v in got["euler"].split())
    assert (cx, ce) == dfp.euler_coeffs(0.5, 0.25)
    assert got["status"].startswith("DFP_ERR_INVALID_ARG")
    assert int(got["ws"]) == dfp.workspace_bytes(dfp.OP_CFG_STEP, 921600, 1, 0, 0, 0, 0, 0)
    assert int(got["ldv"]) == dfp.v_ld(57600, dfp.BF16)
