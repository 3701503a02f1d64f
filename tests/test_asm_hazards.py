"""Wait states after inline-asm matrix instructions (CPU: compiles to gfx950 assembly).

The decode and prefill kernels issue their MFMAs as inline asm, so the
compiler inserts no wait states after them: a VALU instruction, a memory
instruction or another MFMA's A/B operand that reads (or a VALU that
overwrites) the result registers of an MFMA must come enough cycles later,
and the kernels place explicit ``s_nop`` runs for that.  The compiler can
still add reads of its own -- a VALU copy when it moves an accumulator to
other registers, a copy where two branches join -- which nothing in the
source shows.  This test compiles the two sources to assembly with the
library's flags and walks forward from every MFMA, through branches both
ways, counting one wait state per instruction (``s_nop n`` counts n + 1, an
intervening MFMA only 1), and fails if its result registers are touched
before 18 wait states: the requirement of the longest (16-pass) matrix
instruction used here.
"""
import os
import re
import shutil
import subprocess

import pytest

from mla_latent_kv_decode_amd import build as B

NEED = 18
SOURCES = ["decode_mfma.hip", "prefill.hip"]


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _instructions(asm):
    ins, labels = [], {}
    for line in asm.splitlines():
        t = line.strip()
        m = re.match(r"^(\.LBB\d+_\d+):", t)
        if m:
            labels[m.group(1)] = len(ins)
            continue
        if not t or t.startswith((";", ".", "//")) or t.endswith(":"):
            continue
        ins.append(t)
    return ins, labels


def hazards(asm, need=NEED):
    """(mfma, reader, wait states) for every early touch of an MFMA result."""
    ins, labels = _instructions(asm)
    found = set()

    def scan(j, dst, ws, src, seen):
        while j < len(ins) and ws < need:
            if (j, ws) in seen:
                return
            seen.add((j, ws))
            u = ins[j]
            op = u.split()[0]
            if op == "s_endpgm":
                return
            if op == "s_nop":
                ws += int(u.split()[1], 0) + 1
            elif op.startswith("v_mfma"):
                ops = u.split(None, 1)[1].split(",")
                if _regs(",".join(ops[1:3])) & dst:
                    found.add((src, u, ws))
                ws += 1
            elif op.startswith("s_branch"):
                if u.split()[1] not in labels:
                    return
                j = labels[u.split()[1]]
                continue
            elif op.startswith("s_cbranch"):
                ws += 1  # the branch itself, on either path
                if u.split()[1] in labels:
                    scan(labels[u.split()[1]], dst, ws, src, seen)
            else:
                if " " in u and _regs(u.split(None, 1)[1]) & dst:
                    found.add((src, u, ws))
                ws += 1
            j += 1

    for i, t in enumerate(ins):
        if t.startswith("v_mfma"):
            scan(i + 1, _regs(t.split(None, 1)[1].split(",")[0]), 0, t, set())
    return sorted(found, key=lambda f: f[2])


def test_scanner_flags_an_early_read():
    asm = "\n".join([
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
        "s_nop 3",
        "v_mov_b32_e32 v30, v5",          # 4 wait states after: too early
        "s_nop 7", "s_nop 7", "s_nop 7",
        "v_mov_b32_e32 v31, v6",          # 29 after: fine
    ])
    got = hazards(asm)
    assert [(f[1], f[2]) for f in got] == [("v_mov_b32_e32 v30, v5", 4)]
    # through a branch: the read at the target is found as well
    asm2 = "\n".join(["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
                      "s_cbranch_scc1 .LBB0_1", "s_nop 7", "s_nop 7", "s_nop 7", "s_endpgm",
                      ".LBB0_1:", "v_add_f32_e32 v40, v3, v3"])
    assert [f[2] for f in hazards(asm2)] == [1]


@pytest.mark.parametrize("src", SOURCES)
def test_inline_asm_mfma_results_are_not_read_early(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = hazards(out.read_text())
    assert not found, "\n".join(f"{w} wait states: {a}  ->  {b}" for a, b, w in found[:10])
