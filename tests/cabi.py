"""Build helper for ``c_abi_check.c`` (a C program that drives libpdn.so through
its C ABI alone and checks it against the C oracle).  Host code only: gcc,
with the HIP runtime headers and library for device memory and streams."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_abi_check(outdir: str) -> str:
    pkg = os.path.join(ROOT, "gated_delta_rule_77_amd")
    if not os.path.exists(os.path.join(pkg, "libpdn.so")):
        from gated_delta_rule_77_amd import build
        build.build()
    exe = os.path.join(str(outdir), "c_abi_check")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
           os.path.join(ROOT, "tests", "c_abi_check.c"), os.path.join(ROOT, "oracle", "recurrence.c"),
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__", "-L" + pkg, "-lpdn", "-L" + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-fopenmp", "-lm", "-Wl,-rpath," + pkg,
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe
