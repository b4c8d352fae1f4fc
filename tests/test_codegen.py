"""Checks on the generated gfx950 code of the built library (CPU only).

The device code objects are taken from libgdn.so itself (one offload bundle per
source file in its HIP fat-binary section), unbundled and disassembled with the
ROCm LLVM tools, so what is checked is exactly what the tests and the benchmark
run:
- no packed-fp32 instructions (the build turns their selection off);
- every hand-written DPP multiply-add (the prefill's forward substitution) reads
  a DPP source that no vector instruction wrote in the two wait states before
  it, the hazard gfx9 leaves to software for a DPP read after a vector write.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gated_deltanet_recurrence_gdn_amd", "libgdn.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    p = os.path.join(LLVM, name)
    if not os.path.exists(p):
        p = shutil.which(name)
    if p is None:
        pytest.skip(f"{name} is not available")
    return p


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    assert os.path.exists(LIB), "libgdn.so is not built"
    d = tmp_path_factory.mktemp("codegen")
    fat = d / "fatbin.bin"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", LIB], check=True)
    data = fat.read_bytes()
    offs = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert offs, "no offload bundle in libgdn.so"
    text = []
    for n, o in enumerate(offs):
        end = offs[n + 1] if n + 1 < len(offs) else len(data)
        b, c = d / f"b{n}.bin", d / f"c{n}.o"
        b.write_bytes(data[o:end])
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={b}",
                        f"--targets={TARGET}", f"--output={c}"], check=True)
        text.append(subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(c)], check=True,
                                   capture_output=True, text=True).stdout)
    return "\n".join(text)


def _instructions(text):
    """(mnemonic, operands) per instruction; None at every function start."""
    out = []
    for line in text.split("\n"):
        if re.match(r"^[0-9a-f]+ <", line):
            out.append(None)
            continue
        if not line.startswith("\t"):
            continue
        body = line.split("//")[0].strip()
        if not body:
            continue
        parts = body.split(None, 1)
        out.append((parts[0], parts[1] if len(parts) > 1 else ""))
    return out


def _vregs(op):
    m = re.match(r"v\[(\d+):(\d+)\]", op)
    if m:
        return {f"v{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {op} if re.match(r"v\d+$", op) else set()


def test_every_kernel_is_disassembled(disassembly):
    kernels = re.findall(r"^[0-9a-f]+ <(\S+)>:", disassembly, flags=re.M)
    for k in ("verify_chain_kernel", "commit_verify_chain_kernel", "commit_verify_tree_kernel", "commit_kernel",
              "prefill_prepare_kernel", "prefill_scan_kernel", "conv_commit"):
        assert any(k in n for n in kernels), k


def test_no_packed_fp32_instructions(disassembly):
    ins = [i for i in _instructions(disassembly) if i is not None]
    bad = [m for m, _ in ins if m.startswith(("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"))]
    assert not bad, bad[:5]


def dpp_source_hazards(ins):
    """(count of v_fmac_f32_dpp, the ones whose DPP source a vector instruction wrote less than two wait
    states before)."""
    n, bad = 0, []
    for i, x in enumerate(ins):
        if x is None or x[0] != "v_fmac_f32_dpp":
            continue
        n += 1
        src0 = x[1].split(",")[1].strip()
        waits, j = 0, i - 1
        while j >= 0 and waits < 2 and ins[j] is not None:
            m, ops = ins[j]
            if m == "s_nop":
                waits += int(ops.split()[0], 0) + 1
            else:
                if m.startswith("v_") and src0 in _vregs(ops.split(",")[0].strip()):
                    bad.append(f"{m} {ops} -> {x[0]} {x[1]}")
                waits += 1
            j -= 1
    return n, bad


def test_hazard_scan_flags_a_write_just_before():
    snippet = """0000000000001000 <k>:
	v_mov_b32_e32 v7, v1                       // 000000001000: 7E0E0301
	v_fmac_f32_dpp v3, v7, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1 // 000000001004: 76060EFA
	v_add_f32_e32 v9, v1, v1                   // 000000001008: 02121301
	s_nop 1                                    // 00000000100C: BF800001
	v_fmac_f32_dpp v4, v9, v2 row_newbcast:4 row_mask:0xf bank_mask:0xf bound_ctrl:1 // 000000001010: 760812FA
	v_mov_b32_e32 v5, v1                       // 000000001014: 7E0A0301
	v_fmac_f32_dpp v6, v8, v2 row_newbcast:5 row_mask:0xf bank_mask:0xf bound_ctrl:1 // 000000001018: 760C10FA
"""
    n, bad = dpp_source_hazards(_instructions(snippet))
    assert n == 3 and len(bad) == 1 and "v_mov_b32_e32 v7" in bad[0]


def test_dpp_multiply_add_sources_have_their_wait_states(disassembly):
    n, bad = dpp_source_hazards(_instructions(disassembly))
    assert not bad, bad[:3]
    # the prepare kernel's diagonal-block solves: 120 per instance
    assert n > 0 and n % 120 == 0, n
