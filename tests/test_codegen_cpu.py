"""Guards on the gfx950 code of the built library (CPU only; needs a build).

The device code object of every `_build/*.hip.o` is unbundled and
disassembled with the ROCm LLVM tools, and checked for:
* no packed-fp32 VALU forms (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32):
  every HIP source is compiled without them;
* no flat memory instructions: LDS traffic stays ds_*, global traffic
  global_* (a generic pointer turns an LDS store into a flat store, which
  also makes the compiler drain every LDS wait -- this happened once in the
  SQ-format GEMM's decode);
* no scratch (spilled registers) in the FP6/FP4 dual GEMM.
"""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _disassemble(obj, tmp_path):
    base = os.path.join(str(tmp_path), os.path.basename(obj))
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={base}.fb", obj], check=True,
                   capture_output=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", f"--targets={TARGET}", f"--input={base}.fb",
                    f"--output={base}.co", "--unbundle"], check=True, capture_output=True)
    r = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", f"{base}.co"], check=True,
                       capture_output=True, text=True)
    return r.stdout


def _kernels(dis):
    """{mangled kernel name: its disassembly text}"""
    out, name, lines = {}, None, []
    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            if name:
                out[name] = "\n".join(lines)
            name, lines = m.group(1), []
        elif name:
            lines.append(line)
    if name:
        out[name] = "\n".join(lines)
    return out


@pytest.fixture(scope="module")
def objects():
    objs = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
    srcs = glob.glob(os.path.join(ROOT, "outlier_split_mixed_amd", "csrc", "*.hip"))
    if len(objs) != len(srcs) or not os.path.exists(f"{LLVM}/llvm-objdump"):
        pytest.skip("needs the objects of a library build in _build/ and the ROCm LLVM tools")
    return objs


def test_device_code_guards(objects, tmp_path):
    seen = 0
    for obj in objects:
        dis = _disassemble(obj, tmp_path)
        kernels = _kernels(dis)  # (the C-ABI object holds data only)
        for name, text in kernels.items():
            seen += 1
            assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", text), (obj, name, "packed fp32")
            assert not re.search(r"\bflat_(load|store|atomic)", text), (obj, name, "flat memory access")
            if "k_gemm6" in name:
                assert "scratch_" not in text, (obj, name, "register spills")
    assert seen >= 20
