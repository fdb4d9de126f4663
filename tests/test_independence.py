"""The oracle and the HIP path share no code (CPU only).

  * nothing under oracle/ imports the package or reads its sources;
  * nothing in the package imports oracle/ or the input generators;
  * no C/HIP source includes anything from oracle/;
  * the shared input generator (workloads.py) imports neither side and holds
    none of the method's arithmetic (no quantization, packing or sums).
"""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_tensor_activation_amd")
ORACLE = os.path.join(ROOT, "oracle")


def py_files(d):
    for dp, _, fs in os.walk(d):
        for f in fs:
            if f.endswith(".py"):
                yield os.path.join(dp, f)


def imported_modules(path):
    tree = ast.parse(open(path).read(), path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            mods.add(node.module.split(".")[0])
    return mods


def test_oracle_imports_nothing_of_the_package():
    files = list(py_files(ORACLE))
    assert files
    for f in files:
        mods = imported_modules(f)
        assert "bit_tensor_activation_amd" not in mods, f
        assert "csrc" not in open(f).read(), f


def test_package_imports_no_oracle_and_no_generator():
    for f in py_files(PKG):
        mods = imported_modules(f)
        assert "oracle" not in mods and "workloads" not in mods, f


def test_kernel_sources_include_only_their_own_headers():
    inc = re.compile(r'#include\s*[<"]([^>"]+)[>"]')
    for dp, _, fs in os.walk(os.path.join(PKG, "csrc")):
        for f in fs:
            for name in inc.findall(open(os.path.join(dp, f)).read()):
                assert "oracle" not in name, (f, name)
                assert name in {"common.hpp", "btq.h", "hip/hip_runtime.h", "stdint.h",
                                "stddef.h", "float.h", "math.h", "limits.h", "type_traits", "mutex"}, (f, name)


def test_input_generator_is_independent_and_holds_no_codec_arithmetic():
    path = os.path.join(ROOT, "workloads.py")
    mods = imported_modules(path)
    assert not mods & {"oracle", "bit_tensor_activation_amd"}
    src = open(path).read()
    for word in ("rint", "round(", "clamp", "zero_point", "rscale", "nibble"):
        assert word not in src, word
