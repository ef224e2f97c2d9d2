"""CPU check of the built library's device code (gfx950 assembly of this
build, disassembled with the ROCm LLVM tools): no attention kernel contains a
flat memory instruction.  A flat operation counts in both the vector-memory
and the LDS counters, so while one may be outstanding the compiler can wait
for an LDS result only by draining every LDS read, and for its own loads only
with vmcnt(0), which also waits for the tile DMA the kernels issue from inline
assembly.  Every global and LDS access in the kernels therefore goes through
a pointer in its own address space."""
import os
import re
import shutil
import subprocess

import pytest

import decode_attention_kv_attn_amd as A

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _disassembly(tmp_path):
    lib = A.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    if not all(os.path.exists(t) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    fat = tmp_path / "fat.bin"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fat}", lib, str(tmp_path / "lib.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)] + [len(data)]
    assert len(starts) > 1, "no offload bundle in the library"
    text = []
    for i in range(len(starts) - 1):
        part, co = tmp_path / f"b{i}.bin", tmp_path / f"b{i}.co"
        part.write_bytes(data[starts[i]:starts[i + 1]])
        r = subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={part}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        d = subprocess.run([TOOLS[2], "-d", "--no-show-raw-insn", str(co)], capture_output=True, text=True,
                           check=True)
        text.append(d.stdout)
    return "\n".join(text)


def test_attention_kernels_have_no_flat_memory_instructions(tmp_path):
    per_kernel, cur = {}, None
    for line in _disassembly(tmp_path).splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            cur = m.group(1)
            per_kernel.setdefault(cur, 0)
            continue
        if cur is not None and re.search(r"\bflat_\w+", line):
            per_kernel[cur] += 1
    kernels = [k for k in per_kernel if k.startswith("_ZN4attn")]
    assert any("mla_decode_kernel" in k for k in kernels) and any("gqa_mfma_kernel" in k for k in kernels)
    bad = {k: n for k, n in per_kernel.items() if n and k.startswith("_ZN4attn")}
    assert not bad, f"flat memory instructions in {bad}"
