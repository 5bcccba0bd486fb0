"""The attention kernel issues its DPP dot products (v_dot2c_f32_{bf16,f16}
with a row broadcast) and the steps of its all-rows wave maximum
(v_max_f32_dpp) as inline asm, and the compiler does not insert the wait
states such instructions need around code it cannot see into. This test
compiles the kernel source to gfx950 assembly and checks every DPP
instruction (the compiler's own included) against the rules the source
relies on:

  * no VGPR a DPP instruction reads was written by a VALU instruction in the
    two wait states before it;
  * a dot's result is not read by any other instruction within three wait
    states, except by the next dot of the same kind as its accumulator.

No GPU is needed; hipcc cross-compiles."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_fp8_write_amd", "csrc", "decode_attn.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _regs(tok):
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return {f"v{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.fullmatch(r"v\d+", tok) else set()


def _parse(line):
    parts = line.split(None, 1)
    op = parts[0]
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return op, ops


def _violations(asm):
    bad = []
    for kern in re.split(r"\n(?=_Z\S+:)", asm):
        ins = [l.strip() for l in kern.split("\n")]
        ins = [l for l in ins if l and not l.startswith((";", ".")) and not l.endswith(":")]
        for i, line in enumerate(ins):
            op, ops = _parse(line)
            if not op.startswith("v_"):
                continue
            is_dot = op.startswith("v_dot2c_") and op.endswith("_dpp")
            is_dpp = op.endswith("_dpp")
            srcs = set()
            for o in ops[1:]:
                srcs |= _regs(o)
            dst = _regs(ops[0]) if ops else set()
            ws, j = 0, i - 1
            while j >= 0 and ws < 3:
                pop, pops = _parse(ins[j])
                if pop == "s_nop":
                    ws += int(pops[0]) + 1
                    j -= 1
                    continue
                if pop.startswith("v_") and pops:
                    pdst = _regs(pops[0])
                    prev_dot = pop.startswith("v_dot2c_") and pop.endswith("_dpp")
                    if is_dpp and ws < 2 and (srcs & pdst):
                        bad.append(("VALU write -> DPP source", ins[j], line))
                    if prev_dot and pdst:
                        reads = srcs | (dst if is_dot else set())
                        accumulates = is_dot and op == pop and (dst & pdst) and not (srcs & pdst)
                        if (reads & pdst) and not accumulates:
                            bad.append(("dot result read too early", ins[j], line))
                ws += 1
                j -= 1
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_dpp_dot_wait_states(tmp_path):
    out = tmp_path / "attn.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.dirname(SRC), "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    n = len(re.findall(r"v_dot2c_f32_\w+_dpp", asm))
    assert n > 0, "no DPP dot products found"
    assert re.search(r"v_max_f32_dpp", asm), "no fused DPP maximum found"
    bad = _violations(asm)
    assert not bad, f"{len(bad)} wait-state violations, first: {bad[:3]}"
