"""Code placement of the bf16-cache decode kernel's steady-state loop, on the CPU.

The loop's start offset within the kernel changes the batch-4 x 2-query decode by 3-4%
(a measured effect whose cause is not known; see kLoopPadNops in decode.hip).  This test
compiles decode.hip for gfx950 with the library's own flags to assembly, encodes it with
llvm-mc, finds the loop of decode_kernel<false> that holds the step's 68 MFMAs and its
barrier, and checks that it starts at 28 mod 32 bytes from the kernel's 256-byte-aligned
entry.  A change elsewhere in the kernel can move the loop; the failure message says how
many s_nop instructions kLoopPadNops needs then."""

import os
import re
import subprocess

import pytest

from mla_latent_kv_04_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL = "_ZN3mla12_GLOBAL__N_113decode_kernelILb0EEEvNS0_10DecodeArgsE"
LLVM_MC = "/opt/rocm/llvm/bin/llvm-mc"


def _encoded(asm_path):
    """(offset, size, text) of every instruction of KERNEL, and its labels' offsets."""
    r = subprocess.run([LLVM_MC, "-triple", "amdgcn-amd-amdhsa", f"-mcpu={libbuild.ARCH}", "-show-encoding",
                        asm_path], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    off, ins, labels = None, [], {}
    for line in r.stdout.splitlines():
        s = line.strip()
        if s.startswith(KERNEL + ":"):
            off = 0
            continue
        if off is None:
            continue
        if s.startswith(".Lfunc_end"):
            break
        m = re.match(r"^(\.LBB\d+_\d+):", s)
        if m:
            labels[m.group(1)] = off
            continue
        m = re.search(r"encoding: \[([^\]]*)\]", s)
        if m:
            n = len(m.group(1).split(","))
            ins.append((off, n, s.split(";")[0].strip()))
            off += n
    assert ins, f"{KERNEL} not found in the assembly"
    return ins, labels


def test_decode_steady_loop_starts_at_28_mod_32(tmp_path):
    if not os.path.exists(LLVM_MC):
        pytest.skip("llvm-mc not found")
    hipcc = libbuild._hipcc()
    asm = str(tmp_path / "decode.s")
    cmd = [hipcc, *libbuild.HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", libbuild.CSRC,
           "--cuda-device-only", "-S", os.path.join(libbuild.CSRC, "decode.hip"), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    text = open(asm).read()
    # the kernel entry is 256-byte aligned, so offsets from it are offsets mod 256 in memory
    head = text[:text.index(KERNEL + ":")]
    assert re.findall(r"\.p2align\s+(\d+)", head)[-1] == "8"

    ins, labels = _encoded(asm)
    loops = []
    for lab, start in labels.items():
        back = [o for o, n, s in ins if o > start and re.search(r"branch\w*\s+" + re.escape(lab) + r"$", s)]
        if not back:
            continue
        body = [s for o, n, s in ins if start <= o <= back[-1]]
        if sum(s.startswith("v_mfma") for s in body) == 68 and any(s.startswith("s_barrier") for s in body):
            loops.append((lab, start))
    assert len(loops) == 1, f"expected one steady-state loop, found {loops}"
    lab, start = loops[0]
    need = ((28 - start) % 32) // 4
    assert start % 32 == 28, (
        f"steady-state loop {lab} starts at byte {start} of the kernel ({start % 32} mod 32); "
        f"add {need} to kLoopPadNops in decode.hip (mod 8) to put it back at 28 mod 32")
