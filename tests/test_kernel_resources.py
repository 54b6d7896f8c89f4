"""Resources of the built kernels (CPU only): no gfx950 kernel in liblw.so
may use scratch (private segment) memory or spill registers.  A lane array
indexed by a lane-dependent value is placed in scratch, and a spill or such
an array turns into HBM traffic on every launch that no parity test sees.

The device code sits in liblw.so's .hip_fatbin section as clang offload
bundles, one per source file: the magic "__CLANG_OFFLOAD_BUNDLE__", a u64
entry count, then per entry u64 offset, u64 size, u64 triple length and the
triple; offsets are from the bundle's start.  Each gfx950 entry is an AMDGPU
code object whose metadata note lists every kernel's resources."""
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "decode_gemv_amd", "liblw.so")
READELF = "/opt/rocm/llvm/bin/llvm-readelf"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(fatbin: bytes):
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), fatbin)]
    for s in starts:
        pos = s + len(MAGIC)
        (n,) = struct.unpack_from("<Q", fatbin, pos)
        pos += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, pos)
            pos += 24
            triple = fatbin[pos:pos + tlen].decode()
            pos += tlen
            if "gfx950" in triple and size:
                yield fatbin[s + off:s + off + size]


def _kernel_notes(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("liblw.so is not built")
    if not (shutil.which("objcopy") and os.path.exists(READELF)):
        pytest.skip("objcopy or llvm-readelf missing")
    fat = tmp_path / "fat.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", LIB, str(fat)], check=True)
    kernels = {}
    for i, co in enumerate(_code_objects(fat.read_bytes())):
        assert co[:4] == b"\x7fELF"
        p = tmp_path / f"co{i}.o"
        p.write_bytes(co)
        notes = subprocess.run([READELF, "--notes", str(p)], capture_output=True, text=True, check=True).stdout
        # one YAML map per kernel: fields in any order, each map starting at "- .args:" or a field
        for block in re.split(r"\n\s*- \.", notes):
            name = re.search(r"\.name:\s+(\S+)", block)
            if not name or "private_segment_fixed_size" not in block:
                continue
            fields = dict(re.findall(r"\.(\w+):\s+(\d+)\s*$", block, flags=re.M))
            kernels[name.group(1)] = fields
    return kernels


def test_no_kernel_uses_scratch_or_spills(tmp_path):
    kernels = _kernel_notes(tmp_path)
    assert len(kernels) > 300          # every instantiation of every source file
    bad = {k: v for k, v in kernels.items()
           if int(v.get("private_segment_fixed_size", 0)) or int(v.get("vgpr_spill_count", 0))
           or int(v.get("sgpr_spill_count", 0))}
    assert not bad, sorted(bad)[:10]
