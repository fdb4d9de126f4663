"""The C ABI from C (CPU): include/btq.h compiles as C99 with gcc under
-Wall -Werror, the program links libbtq.so, and its calls (size helpers,
status strings, host-side argument checks) behave as the header states."""
import os
import shutil
import subprocess

import pytest

from bit_tensor_activation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_and_library_from_c(tmp_path):
    _lib.load()   # raises if the library has not been built
    exe = str(tmp_path / "abi_from_c")
    lib_dir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(
        ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
         "-L", lib_dir, "-l:libbtq.so", f"-Wl,-rpath,{lib_dir}", "-o", exe],
        check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("all ok")
