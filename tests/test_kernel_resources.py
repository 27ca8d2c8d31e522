"""Register and scratch use of the built gfx950 kernels, read from the code
object metadata of libabgqa.so (no GPU needed).

- The split-KV decode kernels and the direct-to-LDS prefill kernels (every
  path the workloads here take) spill no vector registers and use no private
  (scratch) memory: a spill in a hot loop turns register traffic into memory
  traffic. The register-staged prefill kernels (the fallback for one query
  head per KV head, or caches beyond the direct-to-LDS path's 65536 slots)
  spill 2 to 33 registers at D = 256 and D = 512 (rules); they are held to at
  most that.
- The split-KV decode instantiations compiled for two wavefronts per SIMD
  (head 256 with up to 2 rows per lane group, smaller heads with up to 8) keep
  within the 256 registers that allows, so two workgroups can share a CU.
- The head-512 decode instantiations of eight wavefronts (two per SIMD) fit
  the same 256.
"""
import os
import re
import shutil
import subprocess

import pytest

import additive_bias_gqa_amd as ab

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"


def _kernels(tmp_path):
    """{symbol: {field: int}} from the AMDGPU metadata notes of every gfx950 code object."""
    lib = ab.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    shutil.copy(lib, tmp_path / "lib.so")
    subprocess.run([OBJDUMP, "--offloading", "lib.so"], cwd=tmp_path, check=True, capture_output=True)
    out = {}
    for f in sorted(os.listdir(tmp_path)):
        if not f.endswith("gfx950"):
            continue
        notes = subprocess.run([READELF, "--notes", f], cwd=tmp_path, check=True, capture_output=True,
                               text=True).stdout
        # one YAML list item per kernel, each starting with its .agpr_count
        for item in re.split(r"\n\s*- \.agpr_count:", notes)[1:]:
            name = re.search(r"\.name:\s+(\S+)", item)
            if not name:
                continue
            fields = {"agpr_count": int(item.split("\n", 1)[0].strip())}
            for k in ("vgpr_count", "vgpr_spill_count", "private_segment_fixed_size", "sgpr_count"):
                m = re.search(r"\." + k + r":\s+(\d+)", item)
                fields[k] = int(m.group(1)) if m else 0
            out[name.group(1)] = fields
    return out


@pytest.mark.skipif(not (os.path.exists(OBJDUMP) and os.path.exists(READELF)), reason="ROCm llvm tools not installed")
def test_kernel_registers(tmp_path):
    ks = _kernels(tmp_path)
    decode = {n: f for n, f in ks.items() if "attn_decode_kernel" in n}
    assert len(decode) > 50 and any("attn_prefill_dma_kernel" in n for n in ks)
    for n, f in ks.items():
        if "attn_prefill_kernel" in n or "attn_prefill16_kernel" in n:   # the register-staged fallback
            assert f["vgpr_spill_count"] <= 33 and f["private_segment_fixed_size"] <= 100, (n, f)
            continue
        assert f["vgpr_spill_count"] == 0, f"{n}: {f['vgpr_spill_count']} vector registers spilled"
        assert f["private_segment_fixed_size"] == 0, f"{n}: uses scratch memory"
    # attn_decode_kernel<D, DV, NR, NW, ...>: the mangled template arguments
    arg = re.compile(r"attn_decode_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")
    checked = 0
    for n, f in decode.items():
        D, DV, NR, NW = (int(x) for x in arg.search(n).groups())
        H = max(D, DV)
        two_per_simd = (NW == 4 and ((H <= 256 and NR <= 2) or (H <= 128 and NR <= 8))) or NW == 8
        if two_per_simd:
            checked += 1
            assert f["vgpr_count"] <= 256, f"{n}: {f['vgpr_count']} registers, two wavefronts per SIMD need <= 256"
    assert checked > 20
