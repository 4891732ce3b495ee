"""Checks on the gfx950 machine code of libtriattn.so (CPU only).

The MFMA kernel issues its LDS DMAs (buffer_load_dwordx4 ... lds) from inline
assembly that sets M0 itself, without telling the compiler.  That is only
sound if no compiler-generated instruction in the library reads or writes M0:
this test disassembles the built code object and checks that every M0 write
is one of those sequences and that every LDS DMA is preceded by its own M0
write.
"""
import os
import re
import struct
import subprocess

import pytest

from masked_attention_tri_amd import _native

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
OBJCOPY = "/opt/rocm/llvm/bin/llvm-objcopy"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# instructions that read M0 implicitly besides the LDS DMA
IMPLICIT_M0 = ("s_sendmsg", "s_movrel", "v_movrel", "v_interp", "ds_gws", "ds_append",
               "ds_consume", "s_ttracedata")


def _gfx950_objects(lib, tmp_path):
    fat = tmp_path / "fatbin.bin"
    subprocess.run([OBJCOPY, f"--dump-section=.hip_fatbin={fat}", lib, str(tmp_path / "x.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    out = []
    start = data.find(MAGIC)
    while start >= 0:
        n = struct.unpack_from("<Q", data, start + 24)[0]
        p = start + 32
        for _ in range(n):
            off, size, idlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            tid = data[p:p + idlen].decode()
            p += idlen
            if "gfx950" in tid and size:
                path = tmp_path / f"co{len(out)}.o"
                path.write_bytes(data[start + off:start + off + size])
                out.append(path)
        start = data.find(MAGIC, start + 1)
    return out


@pytest.mark.skipif(not os.path.exists(OBJDUMP) or not os.path.exists(OBJCOPY),
                    reason="ROCm llvm tools not installed")
def test_m0_only_set_by_the_dma_sequences(tmp_path):
    lib = _native.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libtriattn.so not built")
    objs = _gfx950_objects(lib, tmp_path)
    assert objs, "no gfx950 code object in the library"
    n_dma = 0
    for obj in objs:
        asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(obj)], check=True,
                             capture_output=True, text=True).stdout
        ins = []
        for line in asm.splitlines():
            m = re.match(r"\s+([a-z_0-9]+)(\s+[^/]*)?(//.*)?$", line)
            if m and not line.strip().endswith(":"):
                ins.append((m.group(1), (m.group(2) or "").strip()))
        for i, (op, args) in enumerate(ins):
            assert not op.startswith(IMPLICIT_M0), f"{op} reads M0"
            if re.search(r"\bm0\b", args):
                assert op == "s_mov_b32" and args.startswith("m0,"), f"unexpected M0 use: {op} {args}"
                j = i + 1
                while ins[j][0] == "s_nop":
                    j += 1
                assert ins[j][0].startswith("buffer_load") and ins[j][1].endswith("lds"), \
                    f"M0 write not followed by an LDS DMA: {ins[j]}"
            if op.startswith("buffer_load") and args.endswith("lds"):
                n_dma += 1
                j = i - 1
                while ins[j][0] == "s_nop":
                    j -= 1
                assert ins[j][0] == "s_mov_b32" and ins[j][1].startswith("m0,"), \
                    f"LDS DMA without its own M0 write: {ins[j]}"
    assert n_dma > 0
