"""Wait states around the inline-asm MFMAs of the 256 x 224 tile kernels, checked in the
gfx950 assembly the build produces (no GPU needed).

Those kernels issue their MFMAs as inline asm with the accumulators tied to AGPRs, so the
compiler's hazard recognizer does not see them; the kernels keep the required distances by
construction (operands widened or copied several MFMAs before use, s_nop before the
epilogue reads the accumulators).  This test recompiles gemm_a4w4.hip to assembly and checks,
along every control-flow path (fall-through and branch edges, the loop back edge included):
  - no VALU instruction writes a register an MFMA reads (A, B, scales, accumulator) fewer
    than VALU_TO_MFMA wait states before that MFMA;
  - no instruction reads an accumulator register fewer than MFMA_TO_READ wait states after
    the MFMA that wrote it.
The thresholds are conservative bounds on the CDNA3/CDNA4 requirements (a few wait states for
VALU -> MFMA; at most 19 for an MFMA result, 16-pass case).
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNELS = ("gemm_tile224_fp4", "gemm_tile224_fp8")
VALU_TO_MFMA = 4
MFMA_TO_READ = 19


@pytest.fixture(scope="module")
def asm():
    from block_scaled_precision_act_amd import build
    hipcc = build.HIPCC
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = os.path.join(build.CSRC, "gemm_a4w4.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc] + build.COMMON + build.DEVICE + ["--cuda-device-only", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _functions(text, name):
    """{symbol: [instruction lines]} of every instantiation of kernel `name`."""
    out = {}
    for m in re.finditer(r"^(_ZN2mx\d+%s\w+):" % name, text, flags=re.M):
        end = text.index(".Lfunc_end", m.end())
        out[m.group(1)] = text[m.end():end].splitlines()
    return out


def _regs(tok):
    """Registers named by one operand token: ('v'|'a', index) pairs."""
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _parse(lines):
    """Instructions as (mnemonic, operand tokens); labels as ('<label>', [name])."""
    ins = []
    for raw in lines:
        m = re.match(r"^(\.LBB\w*):", raw.strip())
        if m:
            ins.append(("<label>", [m.group(1)]))
            continue
        line = raw.split(";")[0].strip()
        if not line or line.startswith("."):
            continue
        parts = line.split(None, 1)
        ops = [t.strip() for t in parts[1].split(",")] if len(parts) > 1 else []
        ops = [o.split()[0] for o in ops if o]
        ins.append((parts[0], ops))
    return ins


def _wait_states(mn, ops):
    if mn == "s_nop":
        return int(ops[0], 0) + 1
    return 1


def _predecessors(ins):
    """For each index, the indices control can come from: the previous instruction (unless it is
    an unconditional branch or the end of the program) and, at a label, every branch to it."""
    label_at = {ops[0]: i for i, (mn, ops) in enumerate(ins) if mn == "<label>"}
    preds = [[] for _ in ins]
    for i, (mn, ops) in enumerate(ins):
        if i + 1 < len(ins) and mn not in ("s_branch", "s_endpgm"):
            preds[i + 1].append(i)
        if mn.startswith(("s_cbranch", "s_branch")) and ops and ops[0] in label_at:
            preds[label_at[ops[0]]].append(i)
    return preds


def _walk_back(ins, preds, i, limit, hit):
    """Every instruction reachable backwards from i within `limit` wait states: calls
    hit(index, wait states between it and i) for each."""
    seen = {}
    stack = [(p, 0) for p in preds[i]]
    while stack:
        j, ws = stack.pop()
        if ws >= limit or seen.get(j, limit + 1) <= ws:
            continue
        seen[j] = ws
        mn, ops = ins[j]
        if mn != "<label>":
            hit(j, ws)
            ws += _wait_states(mn, ops)
        stack.extend((p, ws) for p in preds[j])


def _check(ins):
    preds = _predecessors(ins)
    problems = []
    for i, (mn, ops) in enumerate(ins):
        if mn.startswith("v_mfma"):
            reads = set()
            for k in (1, 2, 3, 4, 5):
                if k < len(ops):
                    reads |= _regs(ops[k])

            def valu_write(j, ws, reads=reads, mn=mn):
                pm, pops = ins[j]
                if pm.startswith("v_") and not pm.startswith("v_mfma") and pops and _regs(pops[0]) & reads:
                    problems.append("VALU %s writes an operand of %s %d wait states before it" % (pm, mn, ws))
            _walk_back(ins, preds, i, VALU_TO_MFMA, valu_write)
        elif mn.startswith(("v_", "ds_", "global_", "buffer_")) and any(t.startswith("a") for t in ops[1:]):
            reads = set()
            for t in ops[1:]:
                reads |= {r for r in _regs(t) if r[0] == "a"}

            def mfma_write(j, ws, reads=reads, mn=mn):
                pm, pops = ins[j]
                if pm.startswith("v_mfma") and _regs(pops[0]) & reads:
                    problems.append("%s reads the result of %s %d wait states after it" % (mn, pm, ws))
            _walk_back(ins, preds, i, MFMA_TO_READ, mfma_write)
    return problems


@pytest.mark.parametrize("kernel", KERNELS)
def test_inline_asm_mfma_wait_states(asm, kernel):
    funcs = _functions(asm, kernel)
    assert len(funcs) == 2, "expected both VEC instantiations of %s, found %s" % (kernel, list(funcs))
    for sym, lines in funcs.items():
        ins = _parse(lines)
        assert sum(1 for m, _ in ins if m.startswith("v_mfma")) >= 112, sym
        problems = _check(ins)
        assert not problems, "%s:\n%s" % (sym, "\n".join(problems[:10]))


def test_the_checker_catches_a_planted_hazard():
    # a VALU write of an MFMA operand right before it, and an accumulator read right after
    ins = _parse(["\tv_mov_b32_e32 v4, v9", "\tv_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]",
                  "\ts_nop 1", "\tv_accvgpr_read_b32 v20, a2"])
    problems = _check(ins)
    assert len(problems) == 2, problems
