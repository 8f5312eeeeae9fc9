"""Compiled-code guard for the fp8-MFMA attention kernel (CPU only).

V_MFMA_F32_32X32X64_F8F6F4 writes its 16 accumulator registers late: on
MI355X, VALU and memory instructions that read a product's result sooner
than the compiler's minimum wait plus two have returned the accumulator's
previous value, with no error.  A build in which a register copy of the last
d-block's accumulator landed 19 wait states after that product's issue gave
wrong dims 96-127 on the 72-key-page test, and a build with such reads at 20
or more passed every GPU test.  The wait the compiler inserts is its own, and
any change to the kernel's code can move copies and spill stores.  So this
test compiles attn_fp8.hip to AMD assembly with the library's flags and checks
that every such read (with no later matrix product in between, whose issue
waits for the pipe) is at least MIN_WAIT wait states after the product.
"""
import os
import re
import subprocess

import pytest

from chunk_causal_dit_wf_amd import build as wfbuild

MIN_WAIT = 20
STORES = ("scratch_store", "global_store", "buffer_store", "ds_write")


def vregs(tok):
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def split(line):
    s = line.split(";")[0].strip()
    parts = s.split(None, 1)
    return parts[0], (re.findall(r"v\[\d+:\d+\]|v\d+", parts[1]) if len(parts) > 1 else [])


def first_reads(asm):
    """(wait states, instruction, line) of the first non-matrix read of each fp8 product's result
    inside its basic block."""
    lines = asm.split("\n")
    out = []
    for i, l in enumerate(lines):
        s = l.strip()
        if not s.startswith("v_mfma") or "f8f6f4" not in s:
            continue
        dst = vregs(split(s)[1][0])
        dist = 0
        for j in range(i + 1, min(i + 400, len(lines))):
            t = lines[j].strip()
            if not t or t.startswith((".", ";")):
                continue
            if t.endswith(":"):
                break
            op, ops = split(t)
            if op.startswith("s_nop"):
                dist += int(t.split()[1]) + 1
                continue
            if op.startswith(("s_cbranch", "s_branch", "s_endpgm", "v_mfma")):
                break
            srcs = set()
            for k, r in enumerate(ops):
                if k > 0 or op.startswith(STORES):
                    srcs |= vregs(r)
            if srcs & dst:
                out.append((dist, op, j + 1))
                break
            dist += 1
            if ops and not op.startswith(STORES) and vregs(ops[0]) & dst:
                break
    return out


def test_scanner_counts_wait_states():
    asm = "\n".join([
        "\tv_mfma_f32_32x32x64_f8f6f4 v[18:33], v[0:7], v[8:15], v[18:33]",
        "\ts_nop 15",
        "\ts_nop 1",
        "\tv_mov_b64_e32 v[80:81], v[40:41]",
        "\tv_mov_b64_e32 v[96:97], v[32:33]",
    ])
    assert first_reads(asm) == [(19, "v_mov_b64_e32", 5)]


@pytest.mark.timeout(300)
def test_fp8_kernel_reads_products_late_enough(tmp_path):
    out = tmp_path / "attn_fp8.s"
    cmd = [wfbuild.HIPCC] + wfbuild.COMMON + ["-x", "hip", "-S", "--cuda-device-only",
                                              os.path.join(wfbuild.CSRC, "attn_fp8.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert len(re.findall(r"v_mfma_f32_32x32x64_f8f6f4", asm)) > 50, "no fp8 products found in the kernel"
    reads = first_reads(asm)
    assert reads, "no read of a product's result without a later product in between"
    close = [x for x in reads if x[0] < MIN_WAIT]
    assert not close, "fp8 product results read too soon: %s" % close[:5]
