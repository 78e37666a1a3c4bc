"""The machine code libzero.so carries for gfx950, disassembled on the CPU
(this repository's own build): no packed-FP32 arithmetic anywhere (the build
turns the feature off), and the owner update and the fused kernel use the
correctly rounded division expansion and the hardware BF16 conversion that
the bit-exact parity relies on."""
import os
import re
import shutil
import struct
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


def _code_objects(lib_path):
    import bench
    fat = bench._elf_section(lib_path, ".hip_fatbin")
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    pos = fat.find(magic)
    while pos >= 0:
        count, = struct.unpack_from("<Q", fat, pos + len(magic))
        q = pos + len(magic) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fat, q)
            triple = fat[q + 24:q + 24 + tlen]
            q += 24 + tlen
            if b"amdgcn" in triple:
                yield triple.decode(), fat[pos + off:pos + off + size]
        pos = fat.find(magic, pos + len(magic))


@pytest.fixture(scope="module")
def disassembly(libzero, tmp_path_factory):
    from zero_sharded_optimizer_reduce_amd import _lib
    if not (os.path.exists(OBJDUMP) or shutil.which("llvm-objdump")):
        pytest.skip("no llvm-objdump")
    tool = OBJDUMP if os.path.exists(OBJDUMP) else shutil.which("llvm-objdump")
    out = {}
    d = tmp_path_factory.mktemp("co")
    for i, (triple, blob) in enumerate(_code_objects(_lib.LIB_PATH)):
        path = d / f"co{i}.o"
        path.write_bytes(blob)
        r = subprocess.run([tool, "-d", "--demangle", str(path)], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr[-500:]
        out[triple] = r.stdout
    assert out and all("gfx950" in t for t in out)
    return out


def _kernel(text, signature):
    """The instructions of one kernel, from its label to the next blank line."""
    i = text.find(signature)
    assert i >= 0, signature
    return text[i:text.find("\n\n", i)]


def test_no_packed_fp32_arithmetic(disassembly):
    for triple, text in disassembly.items():
        found = sorted(set(re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", text)))
        assert not found, (triple, found)


@pytest.mark.parametrize("signature", ["adam_vec_kernel<0, false, 64>(zero::AdamParams)>:",
                                       "adam_vec_kernel<1, false, 64>(zero::AdamParams)>:",
                                       "fused_vec_kernel<4, 0, false, false, 64>(zero::FusedParams)>:"])
def test_update_kernels_use_correctly_rounded_division_and_hardware_bf16(disassembly, signature):
    for text in disassembly.values():
        k = _kernel(text, signature)
        assert "v_div_fixup_f32" in k and "v_div_scale_f32" in k     # IEEE division expansion
        assert "v_sqrt_f32" in k
        assert "v_cvt_pk_bf16_f32" in k                              # round-to-nearest-even pack
        assert "buffer_store_dwordx4" in k and " nt sc1" in k        # the tile stores with nt | sc1
