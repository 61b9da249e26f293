"""libpdn.so driven from C alone (no Python, no torch in the loop): the program
in ``c_abi_check.c`` allocates device memory and a stream with the HIP runtime,
calls pdn_chunk_fwd (per-channel gates with erase-gate keys and a workspace;
scalar gates with bf16 output) and pdn_decode_step (write-gate keys), checks the
results against the fp64 oracle linked into it, and checks two error codes."""
import subprocess

import pytest

from cabi import build_c_abi_check

pytestmark = pytest.mark.gpu


def test_c_program_drives_the_library(tmp_path):
    exe = build_c_abi_check(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all C-ABI checks passed" in r.stdout
