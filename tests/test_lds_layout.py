"""The rotated byte-table lookups of the QJL score, decode and two-stage score
kernels, and the sign-expansion lookups of the grouped QJL score, use a byte
permute's result as the LDS address itself, which is
right only while the tables start at LDS address 0, i.e. while those
kernels declare no static __shared__ data (dynamic LDS is placed after the
static part).  This reads the built library's gfx950 code objects and checks
that every such kernel has a static LDS size (group_segment_fixed_size) of
zero, so a later static __shared__ declaration fails here instead of
silently reading wrong table entries on the GPU."""
import os
import re
import shutil
import subprocess

import pytest

from kv_cache_compression_kvq_amd import _lib as L

LLVM = "/opt/rocm/llvm/bin"
ADDRESS_ZERO_KERNELS = ("decode_split_kernel", "scores_qjl_kernel", "scores_residual_kernel",
                        "decode_gqa_kernel", "scores_qjl_mfma_kernel")


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def kernel_static_lds(lib_path, tmp_path):
    """{kernel symbol: group_segment_fixed_size} over every gfx950 code object
    bundled in lib_path (one bundle per compiled source)."""
    objcopy, bundler, readelf = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool("llvm-readelf")
    if not (objcopy and bundler and readelf):
        pytest.skip("LLVM binary tools not found")
    fat = tmp_path / "fat.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", lib_path, str(tmp_path / "x.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    out = {}
    for i, a in enumerate(starts):
        b = starts[i + 1] if i + 1 < len(starts) else len(data)
        part, co = tmp_path / f"b{i}.bin", tmp_path / f"b{i}.co"
        part.write_bytes(data[a:b])
        r = subprocess.run([bundler, "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                            f"--output={co}"], capture_output=True, text=True)
        if r.returncode != 0 or not co.exists() or co.stat().st_size == 0:
            continue
        notes = subprocess.run([readelf, "--notes", str(co)], capture_output=True, text=True,
                               check=True).stdout
        for block in re.split(r"\n\s*- \.", notes):
            name = re.search(r"\.name:\s+(\S+)", "." + block)
            size = re.search(r"group_segment_fixed_size:\s+(\d+)", block)
            if name and size:
                out[name.group(1)] = int(size.group(1))
    return out


def test_address_zero_kernels_have_no_static_lds(tmp_path):
    sizes = kernel_static_lds(L.LIB_PATH, tmp_path)
    hits = {k: v for k, v in sizes.items() if any(n in k for n in ADDRESS_ZERO_KERNELS)}
    for n in ADDRESS_ZERO_KERNELS:
        assert any(n in k for k in hits), f"no {n} found in the library's code objects"
    bad = {k: v for k, v in hits.items() if v != 0}
    assert not bad, f"kernels with static LDS (their tables would not start at 0): {bad}"
