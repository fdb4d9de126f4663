"""Generated gfx950 code (CPU): every HIP source is compiled to assembly and
scanned for a hardware hazard and for the register budgets the kernels are
designed around.

A vector-memory store of more than 64 bits of data reads its data registers
after it issues, so a VALU instruction that writes one of those registers
must not come right after it (one wait state is needed). The compiler inserts
that wait state for global stores and for buffer stores with an immediate
scalar offset, but not for buffer stores with a register scalar offset; on
gfx950 such a pair stored the overwritten value in some lanes. The kernels
keep every wide buffer store on an immediate scalar offset; this test checks
the emitted code for the pattern itself, whatever its cause.
"""
import re
import shutil

import pytest

from bit_tensor_activation_amd import build

pytestmark = pytest.mark.skipif(
    shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
    reason="hipcc not found")

WIDE_STORE = re.compile(
    r"^\s*(?:buffer|global|flat)_store_(?:dwordx[34]|b96|b128)\s+(?:[^,]*,\s*)??"
    r"v\[(\d+):(\d+)\]")
VALU_DST = re.compile(r"^\s*v_\S+\s+(?:v\[(\d+):(\d+)\]|v(\d+))\b")


def data_regs(line):
    """The data registers of a wide store, or None. (A buffer store's data
    comes first; a global/flat store's address comes first, its data second.)"""
    s = line.strip()
    ops = [o.strip() for o in s.split(None, 1)[1].split(",")] if " " in s else []
    if not ops:
        return None
    data = ops[1] if s.startswith(("global_", "flat_")) else ops[0]
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", data)
    return set(range(int(m.group(1)), int(m.group(2)) + 1)) if m else None


def is_instruction(s):
    return bool(s) and not s.startswith((";", ".")) and not s.endswith(":")


def hazards(asm_lines):
    """(line number, store, next instruction) for each wide store whose next
    issued instruction is a VALU write to the store's data registers."""
    out = []
    for i, line in enumerate(asm_lines):
        if not WIDE_STORE.match(line):
            continue
        regs = data_regs(line)
        if not regs:
            continue
        j = i + 1
        while j < len(asm_lines) and not is_instruction(asm_lines[j].strip()):
            if asm_lines[j].strip().endswith(":"):   # a label: another path joins here
                break
            j += 1
        if j >= len(asm_lines) or asm_lines[j].strip().endswith(":"):
            continue
        m = VALU_DST.match(asm_lines[j])
        if not m:
            continue
        dst = (set(range(int(m.group(1)), int(m.group(2)) + 1)) if m.group(1)
               else {int(m.group(3))})
        if dst & regs:
            out.append((i + 1, line.strip(), asm_lines[j].strip()))
    return out


def test_scanner_finds_the_pattern():
    bad = ["\tbuffer_store_dwordx4 v[134:137], v140, s[52:55], s20 offen nt",
           "\tv_cndmask_b32_e64 v134, v45, v98, s[18:19]"]
    assert len(hazards(bad)) == 1
    ok_nop = [bad[0], "\ts_nop 0", bad[1]]
    ok_other = [bad[0], "\tv_cndmask_b32_e64 v140, v45, v98, s[18:19]"]
    ok_narrow = ["\tbuffer_store_dwordx2 v[134:135], v140, s[52:55], s20 offen nt", bad[1]]
    glob_bad = ["\tglobal_store_dwordx4 v[32:33], v[28:31], off", "\tv_mov_b32_e32 v29, 0"]
    glob_addr = ["\tglobal_store_dwordx4 v[32:33], v[28:31], off", "\tv_mov_b32_e32 v32, 0"]
    assert hazards(ok_nop) == [] and hazards(ok_other) == [] and hazards(ok_narrow) == []
    assert len(hazards(glob_bad)) == 1 and hazards(glob_addr) == []


@pytest.fixture(scope="module")
def asm_paths(tmp_path_factory):
    return build.device_asm(str(tmp_path_factory.mktemp("asm")))


def kernel_resources(paths):
    """{kernel symbol: {field: value}} from the .amdhsa_kernel descriptors."""
    out = {}
    for p in paths:
        text = open(p).read()
        for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
            fields = dict(re.findall(r"\.amdhsa_(\w+)\s+(\d+)", m.group(2)))
            out[m.group(1)] = {k: int(v) for k, v in fields.items()}
    return out


def test_no_kernel_spills_to_scratch(asm_paths):
    res = kernel_resources(asm_paths)
    assert len(res) > 40
    spills = {k: r["private_segment_fixed_size"] for k, r in res.items()
              if r.get("private_segment_fixed_size", 0)}
    assert not spills, spills


def test_receiver_register_budgets(asm_paths):
    """The receiver's common forms (one set, two entry registers or none, not
    a later group of shards) fit 3 waves per SIMD (at most 168 registers);
    every form fits 2 (at most 256, so no accumulator registers hold
    spills)."""
    res = kernel_resources(asm_paths)
    window = {k: r for k, r in res.items() if "dq_window_kernel" in k}
    assert len(window) >= 96
    for name, r in window.items():
        regs = r["next_free_vgpr"]
        assert regs <= 256, (name, regs)
        m = re.search(r"dq_window_kernelILi(\d)ELi(\d)ELi(\d)ELb(\d)ELb(\d)ELb(\d)E", name)
        assert m, name
        if m.group(2) in ("0", "2") and m.group(4) == "0" and m.group(6) == "0":
            assert regs <= 168, (name, regs)


def test_no_valu_write_to_wide_store_data_on_the_next_instruction(asm_paths):
    paths = asm_paths
    assert paths
    found = {}
    n_wide = 0
    for p in paths:
        lines = open(p).read().splitlines()
        n_wide += sum(1 for l in lines if WIDE_STORE.match(l))
        h = hazards(lines)
        if h:
            found[p] = h[:3]
    assert n_wide > 0          # the scan saw the receiver's wide stores
    assert not found, found
