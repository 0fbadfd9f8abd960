"""The header is plain C: a C11 program compiled with gcc -Wall -Werror -pedantic links
against the library and exercises its host-only paths (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from sparse_graph_attention_02_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_uses_the_abi(tmp_path):
    lib_dir = os.path.dirname(capi.LIB_PATH)
    exe = tmp_path / "abi_smoke"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_smoke.c"),
           "-o", str(exe), capi.LIB_PATH, f"-Wl,-rpath,{lib_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    env["LD_LIBRARY_PATH"] = rocm_lib + os.pathsep + env.get("LD_LIBRARY_PATH", "")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "abi_smoke ok" in r.stdout
