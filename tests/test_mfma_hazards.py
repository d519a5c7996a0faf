"""The library's kernels, compiled for gfx950, never read an MFMA's result registers with a non-MFMA instruction
before the matrix core has finished writing them.

On CDNA the program itself must separate an MFMA from a VALU operation or a memory/LDS instruction that reads the
MFMA's destination registers by enough independent instructions ("wait states"). The compiler counts them inside a
basic block, but a branch or a loop exit between the MFMA and its reader has been seen to leave too few: an LDS
store one instruction after the MFMA on a taken branch, which stored the lanes of the passes not yet written (a
4-row x 16-token block of wrong outputs in a few per cent of calls, more when other kernels ran beside it). The
kernels now wait such reads out explicitly; this test compiles every source to gfx950 assembly and follows every
path from each MFMA (fall-through and branch targets) to check that no reader comes within 8 wait states (the
count the compiler itself places before VALU reads of the 16x16x32 MFMAs used here).
"""
import os
import re
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "nvfp4_weight_only_amd", "csrc")
NEED = 8
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def raw_hazards(asm: str, need: int = NEED):
    """(function, mfma line, reader line, wait states, reader) for every non-MFMA read of an MFMA destination
    register reached within `need` wait states along some path (up to 4 branches deep)."""
    lines = asm.split("\n")
    label_at = {m.group(1): i for i, l in enumerate(lines) for m in [re.match(r"^(\.L\w+):", l)] if m}
    found = []

    def scan(i, dst, budget, depth, origin, func):
        w = 0
        while i < len(lines) and w < budget:
            ins = lines[i].split(";")[0].strip()
            i += 1
            if not ins or ins.endswith(":") or ins.startswith("."):
                continue
            mnem, _, ops = ins.partition(" ")
            ops = ops.strip()
            if mnem == "s_endpgm":
                return
            if mnem.startswith("v_mfma"):
                w += 1
                continue
            if mnem.startswith(("ds_write", "buffer_store", "global_store", "flat_store")):
                srcs = ops
            elif mnem.startswith(("v_", "ds_", "buffer_", "global_", "flat_")):
                srcs = ops.split(",", 1)[1] if "," in ops else ""
            else:
                srcs = ""
            if regs(srcs) & dst:
                found.append((func, origin, i, w, ins))
                return
            if mnem.startswith(("v_", "ds_read", "buffer_load", "global_load")) and "," in ops:
                dst = dst - regs(ops.split(",")[0])  # overwritten: no longer the MFMA's value
                if not dst:
                    return
            if mnem.startswith("s_cbranch") or mnem == "s_branch":
                if ops in label_at and depth < 4:
                    scan(label_at[ops] + 1, dst, budget - w - 1, depth + 1, origin, func)
                if mnem == "s_branch":
                    return
            m = re.match(r"s_nop\s+(\d+)", ins)
            w += int(m.group(1)) + 1 if m else 1

    func = None
    for idx, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):", l)
        if m:
            func = m.group(1)
        ins = l.split(";")[0].strip()
        if ins.startswith("v_mfma"):
            scan(idx + 1, regs(ins.split(None, 1)[1].split(",")[0]), need, 0, idx + 1, func)
    return found


def test_scanner_finds_a_read_behind_a_branch():
    """The scanner itself: an LDS store one instruction after the MFMA on a taken branch is found; the same store
    after 16 wait states is not."""
    bad = """_Zk:
\tv_mfma_f32_16x16x32_bf16 v[6:9], v[10:13], v[14:17], 0
\ts_cbranch_vccnz .LBB0_2
\ts_nop 7
\tv_add_f32_e32 v9, v9, v1
.LBB0_2:
\tds_write_b128 v61, v[6:9]
\ts_endpgm
"""
    assert len(raw_hazards(bad)) == 1
    good = bad.replace("\ts_cbranch_vccnz .LBB0_2\n", "\ts_nop 7\n\ts_nop 7\n\ts_cbranch_vccnz .LBB0_2\n")
    assert raw_hazards(good) == []


@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_no_early_mfma_result_reads(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = raw_hazards(out.read_text())
    assert not found, "\n".join(f"{f} mfma line {o} -> line {i} after {w} wait states: {ins}"
                                for f, o, i, w, ins in found[:20])
