"""Register and scratch use of every kernel in the built library (no GPU).

Reads the gfx950 code objects out of libattnfwd.so's offload bundles and their
AMDGPU metadata notes (llvm-readelf): every kernel must fit 256 VGPRs (two waves
per SIMD for the 512-thread workgroups), spill no registers and use no scratch
memory (which a private array indexed at run time would need).
"""
import os
import re
import shutil
import struct
import subprocess

import pytest

from fp8_causal_prefill_tiled_amd import build

MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _readelf():
    for p in (shutil.which("llvm-readelf"), "/opt/rocm/llvm/bin/llvm-readelf", "/opt/rocm/lib/llvm/bin/llvm-readelf"):
        if p and os.path.exists(p):
            return p
    return None


def _fatbin(lib):
    """The .hip_fatbin section of a shared library (ELF64 little-endian)."""
    with open(lib, "rb") as f:
        d = f.read()
    shoff, = struct.unpack_from("<Q", d, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    sh = [struct.unpack_from("<IIQQQQIIQQ", d, shoff + i * shentsize) for i in range(shnum)]
    strtab = sh[shstrndx]
    names = d[strtab[4]:strtab[4] + strtab[5]]
    for s in sh:
        name = names[s[0]:names.index(b"\0", s[0])]
        if name == b".hip_fatbin":
            return d[s[4]:s[4] + s[5]]
    return b""


def _code_objects(fatbin):
    """gfx950 code objects of every offload bundle in a fat binary."""
    out = []
    pos = fatbin.find(MAGIC)
    while pos >= 0:
        n, = struct.unpack_from("<Q", fatbin, pos + len(MAGIC))
        p = pos + len(MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, p)
            triple = fatbin[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            if "gfx950" in triple:
                out.append(fatbin[pos + off:pos + off + size])
        pos = fatbin.find(MAGIC, pos + 1)
    return out


def _kernels(readelf, co, tmp_path, i):
    path = tmp_path / f"co{i}.elf"
    path.write_bytes(co)
    notes = subprocess.run([readelf, "--notes", str(path)], capture_output=True, text=True, check=True).stdout
    ks = []
    for block in re.split(r"\n\s+- \.agpr_count:", notes)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
        spills = sum(int(x) for x in re.findall(r"\.[sv]gpr_spill_count:\s+(\d+)", block))
        ks.append((name, vgpr, scratch + spills))
    return ks


def test_no_kernel_uses_scratch(tmp_path):
    if not os.path.exists(build.LIB):
        pytest.skip("libattnfwd.so is not built")
    readelf = _readelf()
    if readelf is None:
        pytest.skip("llvm-readelf not found")
    cos = _code_objects(_fatbin(build.LIB))
    # one code object per translation unit with device code
    assert len(cos) == sum(1 for u in build.UNITS if u[1].endswith(".hip"))
    ks = [k for i, co in enumerate(cos) for k in _kernels(readelf, co, tmp_path, i)]
    names = " ".join(k[0] for k in ks)
    for kind in ("fp8_causal_fwd_pair", "fp8_causal_fwdILi128", "fp8_causal_fwdILi192", "bf16_causal_fwdILi192",
                 "rq_stream"):
        assert kind in names, kind
    bad = [k for k in ks if k[2] != 0 or k[1] > 256]
    assert not bad, bad
