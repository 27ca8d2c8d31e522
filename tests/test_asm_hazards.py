"""Wait states before the inline-asm MFMAs of the direct-to-LDS prefill kernel.

The PV products of the 32-row kernels with O^T in the accumulation registers
are inline asm, so the compiler inserts no hazard wait states for them. An
MFMA that reads a register a VALU instruction wrote (the softmax weights P^T,
or an accumulator rewritten by the rescale) needs two wait states in between
(CDNA3/CDNA4 ISA, MFMA dependency rules: VALU write of a VGPR followed by an
MFMA read of it is not interlocked). This test disassembles the gfx950 code of
the built library and checks every such MFMA: scanning back from it (past
other MFMAs: VALU work is interleaved with them), the last VALU write of one
of its source registers must be at least two wait states earlier (s_nop N
counts N + 1, any other instruction 1).
The other direction too: a VALU read of an accumulator (v_accvgpr_read) must
come at least passes + 2 wait states after the MFMA that wrote it; 18 is
taken (16 passes + 2, more than a 32x32x16 MFMA takes).
"""
import os
import re
import shutil
import subprocess

import pytest

import additive_bias_gqa_amd as ab

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MFMA = re.compile(r"v_mfma_f32_32x32x16_bf16 a\[(\d+):(\d+)\], v\[(\d+):(\d+)\], v\[(\d+):(\d+)\], a\[(\d+):(\d+)\]")
DEST = re.compile(r"^(v_\S+)\s+([va])(?:\[(\d+):(\d+)\]|(\d+))\b")
SWAP_SRC = re.compile(r"^v_permlane(?:16|32)_swap\S*\s+v\d+,\s*v(\d+)")
NEED = 2
NEED_READ = 18


def _regs(lo, hi):
    return set(range(int(lo), int(hi) + 1))


def _kernel_bodies(text):
    """{symbol: [instruction text]} for the prefill kernels of one disassembly."""
    bodies, cur = {}, None
    for line in text.splitlines():
        head = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if head:
            cur = head.group(1) if "attn_prefill_dma_kernel" in head.group(1) else None
            if cur:
                bodies[cur] = []
            continue
        if cur and line.startswith("\t"):
            ins = line.strip().split("//")[0].strip()
            if ins:
                bodies[cur].append(ins)
    return bodies


def _min_wait_states(ins):
    """(number of asm-form MFMAs, smallest wait-state distance found)."""
    worst, n = 99, 0
    for i, line in enumerate(ins):
        m = MFMA.match(line)
        if not m:
            continue
        n += 1
        vsrc = _regs(m.group(3), m.group(4)) | _regs(m.group(5), m.group(6))
        asrc = _regs(m.group(7), m.group(8))
        ws = 0
        for k in range(1, 64):
            # VALU work may sit between the MFMAs: scan back past them (each
            # counts one wait state) until the distance no longer matters
            if i - k < 0 or ws >= NEED:
                break
            prev = ins[i - k]
            d = DEST.match(prev)
            if d:
                lo = d.group(3) if d.group(3) is not None else d.group(5)
                hi = d.group(4) if d.group(4) is not None else d.group(5)
                written = _regs(lo, hi)
                if d.group(1).startswith(("v_permlane16_swap", "v_permlane32_swap")):
                    # a lane swap writes both of its operands
                    sw = SWAP_SRC.match(prev)
                    if sw:
                        written |= {int(sw.group(1))}
                if written & (vsrc if d.group(2) == "v" else asrc):
                    worst = min(worst, ws)
                    break
            nop = re.match(r"s_nop (\d+)", prev)
            ws += int(nop.group(1)) + 1 if nop else 1
    return n, worst


def _min_read_wait_states(ins):
    """(VALU reads of an asm MFMA's accumulator found, smallest distance)."""
    worst, n = 999, 0
    for i, line in enumerate(ins):
        m = re.match(r"v_accvgpr_read_b32 v\d+, a(\d+)", line)
        if not m:
            continue
        a, ws = int(m.group(1)), 0
        for k in range(1, 128):
            if i - k < 0:
                break
            prev = ins[i - k]
            mm = MFMA.match(prev)
            if mm and a in _regs(mm.group(1), mm.group(2)):
                n += 1
                worst = min(worst, ws)
                break
            nop = re.match(r"s_nop (\d+)", prev)
            ws += int(nop.group(1)) + 1 if nop else 1
    return n, worst


@pytest.mark.skipif(not os.path.exists(OBJDUMP), reason="ROCm llvm-objdump not installed")
def test_asm_mfma_operands_have_wait_states(tmp_path):
    lib = ab.library_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    shutil.copy(lib, tmp_path / "lib.so")
    subprocess.run([OBJDUMP, "--offloading", "lib.so"], cwd=tmp_path, check=True, capture_output=True)
    checked = 0
    for f in sorted(os.listdir(tmp_path)):
        if not f.endswith("gfx950"):
            continue
        text = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", f], cwd=tmp_path, check=True,
                              capture_output=True, text=True).stdout
        for sym, ins in _kernel_bodies(text).items():
            n, worst = _min_wait_states(ins)
            if n:
                checked += n
                assert worst >= NEED, f"{sym}: an asm MFMA reads a register {worst} wait states after a VALU write"
            n, worst = _min_read_wait_states(ins)
            if n:
                assert worst >= NEED_READ, f"{sym}: an accumulator is read {worst} wait states after its MFMA"
    # the 32-row kernels with accumulation-register O^T are built and checked
    assert checked > 0


def test_scanner_sees_writes_behind_other_mfmas():
    """The scan counts an MFMA between a VALU write and the MFMA reading it as
    one wait state (it does not stop there), and an s_nop N as N + 1."""
    mf = "v_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[{0}:{1}], a[0:15]"
    bad = ["v_pack_b32_f16 v10, v1, v2", mf.format(30, 33), mf.format(8, 11)]
    assert _min_wait_states(bad) == (2, 1)
    ok = ["v_pack_b32_f16 v10, v1, v2", "s_nop 1", mf.format(8, 11)]
    assert _min_wait_states(ok)[1] >= NEED
    far = ["v_pack_b32_f16 v10, v1, v2", mf.format(30, 33), mf.format(40, 43), mf.format(8, 11)]
    assert _min_wait_states(far)[1] >= NEED
    # both operands of a lane swap are written
    swap = ["v_permlane32_swap_b32_e32 v3, v9", mf.format(8, 11)]
    assert _min_wait_states(swap) == (1, 0)
