"""include/wave.h from plain C: a C11 program (tests/c/abi_host.c), compiled
with -pedantic -Werror and linked against libwave.so, builds the Wan2.1-1.3B
7-chunk K=4 progressive plan through the host calls only (no GPU).  Its round
6 must hold R(2), U(3,1), U(4,2), U(5,3), U(6,4), each with the progressive
context phi(j, r) = max(j - r, 0) over every earlier chunk, own slot last
(design-space paper, Table 1 and Figure 2), and the error path must report."""
import os
import shutil
import subprocess

import pytest

from block_causal_attention_wave_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_from_c11_host_calls(tmp_path):
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "abi_host")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
                    "-L", lib_dir, "-lwave", f"-Wl,-rpath,{lib_dir}", "-Wl,-rpath-link,/opt/rocm/lib",
                    "-o", exe], check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    B, K = 7, 4
    head = out[0].split()
    assert int(head[1]) == B + K - 1
    assert int(head[3]) == B * K + (B - 1)  # refreshes R(0..5): chunk 6's clean slot is never read
    want = []
    for i in range(2, 7):
        j = i - 2  # in round 6 chunk i sits at level i - 2: R(2) at 0, then U(3,1) .. U(6,4)
        ctx = [f"{i - r}:{max(j - r, 0)}" for r in range(i, 0, -1)] + [f"{i}:{j}"]
        want.append(f"round 6 node {i} {j} ctx " + " ".join(ctx))
    assert out[1:6] == want
    assert out[6] == f"bad K: rc {_lib.WAVE_ERR_INVALID_ARG} plan null message set"
