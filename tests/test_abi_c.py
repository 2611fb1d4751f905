"""The C ABI from plain C (no GPU): tests/c/abi_from_c.c compiles as C99
against include/ring_attn.h with warnings as errors, links against the
in-tree library, and its host-side calls (version, workspace queries,
argument checks) pass."""
import os
import shutil
import subprocess

import pytest

import blockwise_ring_attention_attn_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    ra.load()   # raises if the library is not built
    exe = tmp_path / "abi_from_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
           "-L", ra.PKG, "-lringattn", "-Wl,-rpath," + ra.PKG, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"
