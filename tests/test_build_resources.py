"""Every gfx950 kernel shipped in libpkv.so runs without scratch memory.

A kernel that needs more registers than the wave has spills them to scratch
(per-lane private memory in HBM), which turns register traffic into memory
traffic on the hot path.  This test reads the AMDGPU code-object metadata of
the built library (the device code of each translation unit sits in one
offload bundle of the .hip_fatbin section) and checks, for every kernel,
that its fixed private segment is 0 bytes and that no VGPR or SGPR was
spilled.  CPU only: it reads the build output, it runs nothing.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_cache_366_amd", "libpkv.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _device_objects(fatbin: bytes):
    """The gfx950 code objects of every offload bundle in a .hip_fatbin
    section.  Bundle layout: magic, entry count (u64), then per entry its
    offset and size (u64, relative to the bundle start), the target triple's
    length (u64) and the triple."""
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), fatbin)]
    objs = []
    for st in starts:
        pos = st + len(MAGIC)
        (n,) = struct.unpack_from("<Q", fatbin, pos)
        pos += 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, pos)
            pos += 24
            triple = fatbin[pos:pos + tlen].decode()
            pos += tlen
            if "gfx950" in triple and size:
                objs.append(fatbin[st + off:st + off + size])
    return objs


def kernel_resources(lib=LIB):
    """{kernel symbol: {metadata key: int}} for every kernel in the library."""
    objcopy, readelf = _tool("llvm-objcopy"), _tool("llvm-readelf")
    if not (objcopy and readelf):
        pytest.skip("llvm-objcopy / llvm-readelf not found")
    res = {}
    with tempfile.TemporaryDirectory() as tmp:
        fb = os.path.join(tmp, "fatbin.bin")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fb}", lib,
                        os.path.join(tmp, "lib.copy")], check=True, capture_output=True)
        with open(fb, "rb") as fh:
            objs = _device_objects(fh.read())
        for i, co in enumerate(objs):
            path = os.path.join(tmp, f"co{i}.elf")
            with open(path, "wb") as fh:
                fh.write(co)
            notes = subprocess.run([readelf, "--notes", path], check=True,
                                   capture_output=True, text=True).stdout
            cur = None
            for line in notes.splitlines():
                m = re.match(r"\s*-?\s*\.(\w+):\s+(\S+)", line)
                if not m:
                    continue
                key, val = m.groups()
                if key == "name" and not val.endswith(".kd"):
                    cur = res.setdefault(val, {})
                elif cur is not None and key in ("private_segment_fixed_size", "vgpr_count",
                                                 "vgpr_spill_count", "sgpr_spill_count"):
                    cur[key] = int(val)
    return res


@pytest.mark.skipif(not os.path.exists(LIB), reason="libpkv.so is not built")
def test_no_kernel_uses_scratch():
    res = kernel_resources()
    kernels = [k for k in res if "kernel" in k]
    # every translation unit's kernels are found (decode, prefill, reduce,
    # cache operations)
    for part in ("decode_wave_kernel", "decode_mfma_kernel", "prefill_mfma_kernel",
                 "reduce_kernel", "reshape_and_cache_kernel", "copy_blocks_kernel"):
        assert any(part in k for k in kernels), part
    bad = {k: v for k, v in res.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)
           or v.get("sgpr_spill_count", 0)}
    assert not bad, "kernels with scratch or spills:\n" + "\n".join(
        f"{k}: {v}" for k, v in sorted(bad.items()))
