"""Static check of the matrix-core result hazard in this library's own gfx950
assembly (CPU only: the kernels are compiled to assembly, nothing runs).

The hardware does not interlock a vector-ALU, LDS or memory instruction
against the result of a matrix-core (XDL) instruction: the program must leave
enough independent issue slots in between.  CDNA3 asks NumPasses + 3 slots for
an XDL write followed by another instruction reading or writing the same
registers; gfx950 asks one more for ops of four or more passes.  The compiler
pads most such accesses with NumPasses + 4 but some with only NumPasses + 3
(an accumulator read 19 slots after a 32x32x64 E4M3 op was seen to miss that
op's contribution), so the kernels pad explicitly after their K loops.  This
test walks every path leaving every MFMA (fall-through and branch targets)
and fails if any access to its destination registers comes sooner than
NumPasses + 4 slots.  Pass counts are the issue intervals of independent
back-to-back ops on gfx950 (4 cycles a pass)."""
import importlib.util
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_linear_layers_token_amd", "csrc")
KERNELS = ["gemm_large.hip", "gemm_packed.hip", "gemm_small.hip", "linear.hip", "linear_tokens.hip", "weight_only.hip", "gemv.hip",
           "quant_act.hip"]

PASSES = {
    "v_mfma_f32_32x32x64_f8f6f4": 16,   # E4M3 operands
    "v_mfma_f32_16x16x128_f8f6f4": 8,
    "v_mfma_i32_32x32x32_i8": 8,
    "v_mfma_i32_16x16x64_i8": 4,
    "v_mfma_f32_32x32x16_bf16": 8,
    "v_mfma_f32_16x16x32_bf16": 4,
}

_REG = re.compile(r"\b([av])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _parse(asm):
    """-> (instructions [(mnemonic, operand text)], label -> instruction index)."""
    ins, labels = [], {}
    for raw in asm.splitlines():
        t = raw.split(";")[0].strip()
        if not t or t.startswith("."):
            if t.endswith(":"):
                labels[t[:-1]] = len(ins)
            continue
        if t.endswith(":"):
            labels[t[:-1]] = len(ins)
            continue
        op = t.split()[0]
        ins.append((op, t[len(op):]))
    return ins, labels


def _slots(op, rest):
    if op == "s_nop":
        return int(rest.strip(), 0) + 1
    return 1


def violations(asm):
    """[(mfma mnemonic, slots, accessing instruction, mfma index)] with slots < NumPasses + 4."""
    ins, labels = _parse(asm)
    bad = []
    for i, (op, rest) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        if op not in PASSES:
            raise AssertionError(f"unknown matrix-core op {op}: add its pass count")
        need = PASSES[op] + 4
        dst = _regs(rest.split(",")[0])
        seen = {}
        stack = [(i + 1, 0)]
        while stack:
            j, ws = stack.pop()
            while j < len(ins) and ws < need:
                if seen.get(j, -1) >= ws:
                    break
                seen[j] = ws
                o, r = ins[j]
                parts = r.split(",")
                if o.startswith("v_mfma"):
                    srcab = _regs(",".join(parts[1:3]))
                    srcc = _regs(parts[3]) if len(parts) > 3 else set()
                    if srcab & dst:
                        bad.append((op, ws, o + r, i))
                        break
                    if _regs(parts[0]) & dst or srcc & dst:
                        break        # chained accumulation: interlocked; the new op is checked at its own site
                elif _regs(r) & dst:
                    bad.append((op, ws, o + r, i))
                    break
                if o in ("s_endpgm", "s_setpc_b64"):
                    break
                ws += _slots(o, r)
                if o == "s_branch":
                    j = labels[r.strip()]
                    continue
                if o.startswith("s_cbranch"):
                    stack.append((labels[r.split(",")[-1].strip()], ws))
                j += 1
    return bad


def _load_build():
    spec = importlib.util.spec_from_file_location("qlin_build", os.path.join(ROOT, "quantized_linear_layers_token_amd",
                                                                            "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _asm(src, outdir, flags, hipcc):
    out = os.path.join(outdir, os.path.splitext(src)[0] + ".s")
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    with open(out) as f:
        return f.read()


def test_scanner_flags_a_short_gap():
    # the scanner itself: 19 slots after a 16-pass op is one short, 20 is enough
    def prog(nops):
        return ("\tv_mfma_f32_32x32x64_f8f6f4 a[0:15], v[0:7], v[8:15], a[0:15]\n" + "\ts_nop 0\n" * nops +
                "\tv_accvgpr_read_b32 v20, a15\n\ts_endpgm\n")
    assert violations(prog(19)) and not violations(prog(20))
    # a taken branch is followed; a chained MFMA ends the path
    br = ("\tv_mfma_i32_16x16x64_i8 v[0:3], v[4:7], v[8:11], v[0:3]\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 15\n"
          ".LBB0_2:\n\tv_add_u32_e32 v20, v1, v20\n\ts_endpgm\n")
    assert violations(br)
    chain = ("\tv_mfma_i32_16x16x64_i8 v[0:3], v[4:7], v[8:11], v[0:3]\n"
             "\tv_mfma_i32_16x16x64_i8 v[0:3], v[12:15], v[8:11], v[0:3]\n\ts_nop 7\n\tv_add_u32_e32 v20, v1, v20\n")
    assert not violations(chain)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not installed")
def test_every_mfma_result_access_is_padded(tmp_path):
    b = _load_build()
    hipcc = b.hipcc()
    flags = [f for f in b.CFLAGS if f not in ("-fPIC",)]
    with ThreadPoolExecutor(min(len(KERNELS), os.cpu_count() or 1)) as ex:
        texts = list(ex.map(lambda s: _asm(s, str(tmp_path), flags, hipcc), KERNELS))
    report = []
    nmfma = 0
    for src, text in zip(KERNELS, texts):
        nmfma += sum(1 for op, _ in _parse(text)[0] if op.startswith("v_mfma"))
        for op, ws, what, _ in violations(text)[:5]:
            report.append(f"{src}: {op} -> {what.strip()} after {ws} slots (need {PASSES[op] + 4})")
    assert nmfma > 1000, "no matrix-core code found"
    assert not report, "\n".join(report)
