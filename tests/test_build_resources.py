"""The compiled kernels' resource metadata (CPU only; reads the built library).

Every kernel of libdg.so must run without scratch memory: no register spills
and no private arrays demoted to the stack (a demoted array made one attention
variant 25x slower while its results stayed correct, so only this check
catches it). The attention kernel at head_dim 64 must also fit three waves per
SIMD (its registers bound the occupancy it was tuned for).

The gfx950 code objects are taken from the library's offload bundles and their
AMDGPU metadata notes read with llvm-readelf.
"""
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "dense_gemm_07_amd", "lib", "libdg.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


def code_objects(fatbin):
    """The gfx950 code objects of a sequence of offload bundles: each bundle
    is the magic, an entry count, then (offset, size, triple length, triple)
    per entry, offsets relative to the bundle's start."""
    out = []
    start = fatbin.find(MAGIC)
    while start != -1:
        count = struct.unpack_from("<Q", fatbin, start + len(MAGIC))[0]
        q = start + len(MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, q)
            q += 24
            triple = fatbin[q:q + tlen].decode()
            q += tlen
            if "gfx950" in triple and size:
                out.append(fatbin[start + off:start + off + size])
        start = fatbin.find(MAGIC, start + 1)
    return out


def kernels(tmp_path):
    objcopy, readelf = tool("llvm-objcopy"), tool("llvm-readelf")
    if not os.path.exists(LIB) or not objcopy or not readelf:
        pytest.skip("built library or llvm tools missing")
    fat = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fat}", LIB, str(tmp_path / "lib.so")], check=True)
    found = {}
    for i, co in enumerate(code_objects(fat.read_bytes())):
        path = tmp_path / f"co{i}.o"
        path.write_bytes(co)
        notes = subprocess.run([readelf, "--notes", str(path)], check=True, capture_output=True, text=True).stdout
        for block in notes.split("  - .agpr_count:")[1:]:
            fields = dict(re.findall(r"^\s+\.(\w+):\s+(\S+)\s*$", block, re.M))
            found[fields["name"]] = fields
    return found


def test_no_kernel_uses_scratch(tmp_path):
    ks = kernels(tmp_path)
    assert len(ks) > 100, len(ks)  # every unit's instantiations were found
    bad = {n: (f["private_segment_fixed_size"], f["vgpr_spill_count"], f["uses_dynamic_stack"])
           for n, f in ks.items()
           if f["private_segment_fixed_size"] != "0" or f["vgpr_spill_count"] != "0"
           or f["uses_dynamic_stack"] != "false"}
    assert not bad, f"kernels with scratch memory or spills (bytes per lane, spilled VGPRs, dynamic stack): {bad}"


def test_attention_head_dim_64_fits_three_waves_per_simd(tmp_path):
    ks = kernels(tmp_path)
    att = {n: int(f["vgpr_count"]) for n, f in ks.items() if "attn_fwd" in n and "Li64E" in n}
    assert len(att) == 4, sorted(att)  # bf16/f16 x causal or not
    assert all(v <= 168 for v in att.values()), att  # 512 registers / 3 waves, in granules of 8
