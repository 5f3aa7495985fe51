"""The prefill ring's global-to-LDS copies set m0 with a scalar add inside
inline assembly; that add also writes SCC (the scalar carry / compare bit).
The statements declare SCC clobbered, so the compiler never carries a value
in SCC across them (for example between the two halves of a 64-bit address
add, where a lost carry leaves the pointer 4 GiB low). This test reads the
gfx950 code of the built library (disassembled with ROCm's llvm-objdump) and
checks, after every such copy, that the next instruction touching SCC
writes it rather than reads it. CPU only."""
import os
import re
import shutil
import subprocess

import pytest

from weight_only_int4_unpack_amd import build

LLVM = "/opt/rocm/llvm/bin"
READS = ("s_addc_u32", "s_subb_u32", "s_cbranch_scc0", "s_cbranch_scc1", "s_cselect_b32",
         "s_cselect_b64", "s_cmovk_i32", "s_cmov_b32", "s_cmov_b64")
WRITES = re.compile(r"s_(add|sub)_[iu]32|s_(addc|subb)_u32|s_cmp|s_(and|or|xor|andn2|orn2|nand|nor|xnor|not)_b|"
                    r"s_(lshl|lshr|ashr)|s_bfe|s_(min|max)_|s_abs|s_bcnt|s_absdiff|s_mul_hi")
END = re.compile(r"s_cbranch|s_branch|s_endpgm|s_setpc|s_swappc")


def _disassemble(tmp_path):
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in tools) or not os.path.exists(build.LIB):
        pytest.skip("ROCm LLVM tools or the built library are missing")
    fat, co = str(tmp_path / "fatbin"), str(tmp_path / "gfx950.co")
    subprocess.run([tools[0], "--dump-section", f".hip_fatbin={fat}", build.LIB,
                    str(tmp_path / "copy.so")], check=True, capture_output=True)
    subprocess.run([tools[1], "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--input={fat}", f"--output={co}"], check=True, capture_output=True)
    out = subprocess.run([tools[2], "-d", "--no-show-raw-insn", co], check=True, capture_output=True,
                         text=True).stdout
    return [l.split("//")[0].strip() for l in out.splitlines()]


def test_lds_copies_keep_scc_dead(tmp_path):
    lines = _disassemble(tmp_path)
    copies = [i for i, l in enumerate(lines) if l.startswith("s_add_u32 m0,")]
    assert len(copies) > 100          # the ring kernels' copies are in the library
    bad = []
    for i in copies:
        for l in lines[i + 1:]:
            op = l.split(" ")[0]
            if op.startswith(READS):
                bad.append(lines[i - 2:i + 1] + [l])
                break
            if WRITES.match(op) or END.match(op):
                break
    assert not bad, f"{len(bad)} copies with SCC read after them, e.g. {bad[:2]}"
