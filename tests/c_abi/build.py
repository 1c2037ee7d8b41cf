"""Compile the C-ABI test driver (tests/c_abi/a2av_c_driver.c) with gcc
against the built library and the C oracle; the executable lands beside the
source.  Test infrastructure: called by the package build entry point."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "a2av_c_driver.c")
EXE = os.path.join(HERE, "a2av_c_driver")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), SRC,
           "-o", tmp,
           "-L" + os.path.join(ROOT, "all_movement_amd"), "-la2av",
           "-L" + os.path.join(ROOT, "oracle"), "-la2av_oracle",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../all_movement_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(tmp, EXE)
    return EXE
