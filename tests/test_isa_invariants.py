"""Invariants of the gfx950 machine code the library is built into, checked on
the disassembly of each compiled object (no GPU needed):

* M0 is written only to address an LDS-direct load: every instruction that
  names M0 is `s_mov_b32 m0, <sgpr>` immediately followed by a
  `buffer_load_dword* ... lds`.  The loads are written as inline assembly
  (so the compiler neither counts them nor makes later LDS reads wait for
  them) and set M0 themselves; this test turns the assumption that no other
  code in the kernels keeps a value in M0 into a checked property.
* No packed FP32 arithmetic (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the
  build disables the feature for all device code.

The objects are the in-tree build's (precision_dense_linear_amd/_build/*.o);
each carries its device code as an offload bundle, unbundled here with the
ROCm LLVM tools."""
import glob
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "precision_dense_linear_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
OBJECTS = sorted(glob.glob(os.path.join(BUILD, "*.o")))


def disassemble(obj: str, tmp: str) -> list:
    """(mnemonic, operands) of every instruction of obj's gfx950 code."""
    fat = os.path.join(tmp, "fatbin")
    dev = os.path.join(tmp, "device.o")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat, obj], check=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o", "--targets=" + TARGET,
                    "--input=" + fat, "--output=" + dev, "--unbundle"], check=True)
    text = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", dev], check=True,
                          stdout=subprocess.PIPE, text=True).stdout
    out = []
    for line in text.splitlines():
        m = re.match(r"\s+([a-z][a-z0-9_]*)\b\s*(.*?)\s*(//|$)", line)
        if m and not line.lstrip().startswith(("Disassembly", "<")):
            out.append((m.group(1), m.group(2)))
    return out


def test_build_objects_present():
    assert OBJECTS, "no objects under %s: build the library first (__graft_entry__.build())" % BUILD


@pytest.mark.parametrize("obj", OBJECTS, ids=[os.path.basename(o) for o in OBJECTS])
def test_machine_code_invariants(obj):
    with tempfile.TemporaryDirectory() as tmp:
        ins = disassemble(obj, tmp)
    assert ins, "%s: no instructions disassembled" % obj
    m0_writes = 0
    for i, (op, args) in enumerate(ins):
        assert not re.match(r"v_pk_(add|mul|fma)_f32$", op), "%s: packed FP32 instruction %s" % (obj, op)
        if re.search(r"\bm0\b", args):
            assert op == "s_mov_b32" and args.startswith("m0,"), "%s: M0 used by %s %s" % (obj, op, args)
            nop, nargs = ins[i + 1]
            assert nop.startswith("buffer_load_dword") and re.search(r"\blds\b", nargs), (
                "%s: M0 write not followed by an LDS-direct load: %s" % (obj, (nop, nargs)))
            m0_writes += 1
    name = os.path.basename(obj)
    if name in ("gemm.o", "gemm_skinny.o", "attention.o"):
        assert m0_writes > 0, "%s: expected LDS-direct loads" % name
