"""The single-launch cascade's dealing of block roles, checked on the CPU.

`cascade_role` (in the matrix-core kernel source) tells each block of the one
grid whether it is a prefix or a suffix block and which one. The test takes the
function's text from that source, drops its device qualifiers and builds it with
g++ into tests/host/cascade_dealing.cpp, which checks that the dealing is a
bijection onto the prefix and suffix indices for every pair of counts in a range,
and that 256 + 256 blocks give every compute unit one block of each role under
the dispatch order the dealing assumes. Runs without a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_fdec_amd", "csrc", "split_kv_mfma.hip")
HOST = os.path.join(ROOT, "tests", "host")


def extract_cascade_role(text: str) -> str:
    m = re.search(r"^__device__ __forceinline__ void cascade_role\(.*?^\}\n", text, re.S | re.M)
    assert m, "cascade_role not found in the kernel source"
    body = m.group(0).replace("__device__ __forceinline__ ", "static inline ", 1)
    assert "__" not in body.split("\n", 1)[1], "device-only code inside cascade_role"
    return body


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_cascade_dealing_is_a_bijection_and_pairs_roles(tmp_path):
    with open(SRC) as f:
        (tmp_path / "cascade_role_extracted.inc").write_text(extract_cascade_role(f.read()))
    exe = str(tmp_path / "cascade_dealing")
    r = subprocess.run(["g++", "-std=c++17", "-O2", f"-I{tmp_path}", os.path.join(HOST, "cascade_dealing.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "dealing ok" in r.stdout, r.stdout[-3000:] + r.stderr[-2000:]
