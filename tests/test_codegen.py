"""Checks on the gfx950 assembly of the kernels (hipcc only, no GPU).

Three properties of the generated code that neither the compiler nor a CPU
test would otherwise catch; each would only show on a GPU, as wrong results:

- The compiler inserts no wait states before inline asm.  The asm rounding
  `v_cvt_pk_bf16_f32 vD, 0, vS` (the only source of that form: the compiler's
  own conversions take two registers) must therefore read a register written
  by ordinary VALU arithmetic, never by an MFMA or a transcendental
  instruction, whose results need wait states before a VALU read.
- A bf16-pair operand of `v_dot2c_f32_bf16` that the compiler encodes as an
  inline float constant is applied by the hardware as that 32-bit float, not
  as the bf16 pair meant (the pair (-1, 0) became -1.0, i.e. (0, -1)).  Every
  such operand must be a register or a literal.
- No packed fp32 VALU instructions are generated (the build disables them).
"""
import os
import re
import shutil
import subprocess

import pytest

from chunkwise_gated_linear_amd import build as gla_build

SOURCES = ["gla_walk_bf16.hip", "gla_kernels.hip"]
TRANSCENDENTAL = re.compile(r"^v_(exp|log|rcp|rsq|sqrt|sin|cos)_")
# first operand is not written (stores, compares into SGPRs or vcc, lane reads)
NO_VECTOR_DEST = re.compile(r"^(s_|v_cmp|v_readlane|v_readfirstlane|ds_write|ds_store|buffer_store|"
                            r"global_store|scratch_store|flat_store)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in SOURCES:
        path = os.path.join(str(d), src + ".s")
        res = subprocess.run(gla_build.device_asm_command(src, path), capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(path) as f:
            out[src] = f.read().splitlines()
    return out


def _instructions(lines):
    """(index, mnemonic, operand text) of each instruction line; labels give None."""
    for n, line in enumerate(lines):
        if re.match(r"^[.\w$]+:", line):
            yield n, None, None
            continue
        if not line.startswith("\t") or line.startswith("\t.") or line.startswith("\t;"):
            continue
        parts = line.split(None, 1)
        yield n, parts[0], (parts[1].split(";")[0] if len(parts) > 1 else "")


def _vregs(operand):
    operand = operand.strip()
    m = re.fullmatch(r"v(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def test_asm_rounding_reads_plain_valu_results(asm):
    lines = asm["gla_walk_bf16.hip"]
    insts = list(_instructions(lines))
    checked = 0
    for pos, (n, mn, ops) in enumerate(insts):
        if mn != "v_cvt_pk_bf16_f32":
            continue
        m = re.fullmatch(r"\s*v\d+, 0, v(\d+)\s*", ops)
        if not m:
            continue
        src = int(m.group(1))
        writer = None
        for _, wmn, wops in reversed(insts[:pos]):
            assert wmn is not None, f"line {n + 1}: the input v{src} is written in another basic block"
            if NO_VECTOR_DEST.match(wmn):
                continue
            if src in _vregs(wops.split(",")[0]):
                writer = wmn
                break
        assert writer is not None, f"line {n + 1}: no writer of v{src}"
        assert not writer.startswith("v_mfma"), f"line {n + 1}: v{src} comes straight from {writer}"
        assert not TRANSCENDENTAL.match(writer), f"line {n + 1}: v{src} comes straight from {writer}"
        checked += 1
    assert checked > 0, "the asm rounding form is no longer generated; update this test"


@pytest.mark.parametrize("src", SOURCES)
def test_bf16_dot_operands_are_registers_or_literals(asm, src):
    for n, mn, ops in _instructions(asm[src]):
        if mn is None or not re.match(r"^v_dot2c?_f32_bf16", mn):
            continue
        for operand in ops.split(",")[1:]:
            operand = operand.strip()
            assert re.fullmatch(r"[vs]\d+|[vs]\[\d+:\d+\]|0x[0-9a-fA-F]+", operand), \
                f"{src} line {n + 1}: {mn} {ops.strip()}: operand {operand} is an inline constant"


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32_instructions(asm, src):
    bad = [l.strip() for l in asm[src] if re.match(r"^\s+v_pk_(add|mul|fma)_f32", l)]
    assert not bad, f"{src}: {bad[:3]}"
