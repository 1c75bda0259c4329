"""Compile the HIP library (gfx950) in place: libverify_attn.so next to this file."""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "verify_attn.hip")
LIB = os.path.join(HERE, "libverify_attn.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Werror",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMAs the compiler emits keep their accumulators in VGPRs: the AGPRs are
    # reserved for the partial kernel's output accumulators (asm MFMAs)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE,
]


def check_registers(extra=()) -> dict:
    """Compile the device code to assembly and check the partial kernels'
    register allocation: no spills, and the AGPRs of the output accumulators
    (the asm MFMAs rely on the compiler never touching them)."""
    with tempfile.TemporaryDirectory() as tmp:
        asm = os.path.join(tmp, "verify_attn.s")
        cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC", "-Werror")], *extra,
               "--cuda-device-only", "-S", SRC, "-o", asm]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc -S failed ({res.returncode}): {' '.join(cmd)}")
        text = open(asm).read()
    meta = text[text.index("amdhsa.kernels"):]
    info = {}
    for block in meta.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        info[name] = {
            "agpr": int(block.split()[0]),
            "vgpr_spill": int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1)),
            "sgpr_spill": int(re.search(r"\.sgpr_spill_count:\s+(\d+)", block).group(1)),
        }
    # bf16 kernel: 256 output accumulators; fp32 kernel: 128 (the compiler may
    # round the AGPR block up). Neither may spill.
    # small-row kernel: its query block (72 or 144 registers) in AGPRs.
    need = {"verify_attn_partial_kernelILb0ELb0E": lambda n: n == 256,  # several sequences
            "verify_attn_partial_kernelILb0ELb1E": lambda n: n == 256,  # several, idle waves
            "verify_attn_partial_kernelILb1ELb0E": lambda n: n == 256,  # one sequence
            "verify_attn_partial_kernelILb1ELb1E": lambda n: n == 256,  # one, idle waves
            "verify_attn_partial_small_kernelILi1E": lambda n: n >= 72,
            "verify_attn_partial_small_kernelILi2E": lambda n: n >= 144,
            "verify_attn_f32_partial_kernelE": lambda n: n >= 128}
    for kname, agpr_ok in need.items():
        found = [v for k, v in info.items() if kname in k]
        if len(found) != 1:
            raise RuntimeError(f"{kname} not found in the assembly metadata: {sorted(info)}")
        p = found[0]
        if p["vgpr_spill"] or p["sgpr_spill"] or not agpr_ok(p["agpr"]):
            raise RuntimeError(f"{kname} register allocation changed: {p}")
    check_mfma_hazards(text, "verify_attn_f32_partial_kernel")
    for kernel in ("verify_attn_partial_small_kernelILi1E", "verify_attn_partial_small_kernelILi2E"):
        check_mfma_hazards(text, kernel)
        check_asm_b_operands_invariant(text, kernel)
        check_asm_mfma_result_reads(text, kernel)
    return info


def _regs(tok, kind="v"):
    """Register numbers of one operand token of register file `kind` ("v" or "a")."""
    tok = tok.split()[0] if tok.split() else tok  # drop modifiers such as "offset:16"
    m = re.match(kind + r"\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(kind + r"(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vregs(tok):
    return _regs(tok, "v")


def _operands(line):
    return [t.strip() for t in line.split(None, 1)[1].split(",")] if " " in line else []


def check_mfma_hazards(text, kernel):
    """The asm MFMAs of `kernel` with an AGPR operand carry no wait states of
    their own: require that none of the two instructions issued before one of
    them is a VALU instruction writing one of its source registers (VGPR or
    AGPR)."""
    # the kernel's entry label: a line "<mangled name containing `kernel`>:"
    m = re.search(r"^(_Z\S*" + re.escape(kernel) + r"\S*):", text, flags=re.M)
    if not m:
        raise RuntimeError(f"{kernel}: entry label not found in the assembly")
    body = text[m.end():]
    body = body[:body.index("s_endpgm")]
    ins = [l.split(";")[0].strip() for l in body.splitlines()]
    ins = [l for l in ins if l and not l.startswith(".") and not l.endswith(":")]
    for i, line in enumerate(ins):
        if not (line.startswith("v_mfma") and " a[" in line):
            continue
        ops = _operands(line)
        src = {("v", r) for t in ops[1:] for r in _regs(t, "v")} | {("a", r) for t in ops[1:] for r in _regs(t, "a")}
        issued, k = 0, i - 1
        while k >= 0 and issued < 2:
            prev = ins[k]
            k -= 1
            if prev.startswith("s_nop"):
                issued += int(prev.split()[1]) + 1
                continue
            if prev.startswith("s_waitcnt"):
                continue
            issued += 1
            if prev.startswith("v_") and not prev.startswith("v_mfma"):
                d = _operands(prev)[0]
                dst = {("v", r) for r in _regs(d, "v")} | {("a", r) for r in _regs(d, "a")}
                if dst & src:
                    raise RuntimeError(f"{kernel}: VALU write right before an asm MFMA source: "
                                       f"{prev!r} -> {line!r}")


def _kernel_body(text, kernel):
    m = re.search(r"^(_Z\S*" + re.escape(kernel) + r"\S*):", text, flags=re.M)
    if not m:
        raise RuntimeError(f"{kernel}: entry label not found in the assembly")
    body = text[m.end():]
    body = body[:body.index("s_endpgm")]
    ins = [l.split(";")[0].strip() for l in body.splitlines()]
    return [l for l in ins if l and not l.startswith(".") and not l.endswith(":")]


def check_asm_b_operands_invariant(text, kernel):
    """The QK MFMAs of the small-row kernel read the query from AGPRs (their B
    operand) for the whole split: require that no instruction between
    the first and the last of them writes one of those AGPRs (a copy into an
    AGPR right before an asm MFMA would need wait states the compiler does not
    know to insert)."""
    ins = _kernel_body(text, kernel)
    mf = [i for i, l in enumerate(ins) if l.startswith("v_mfma") and ", a[" in l]
    if not mf:
        raise RuntimeError(f"{kernel}: no asm MFMA with an AGPR operand found")
    b_regs = set()
    for i in mf:
        b_regs |= _regs(_operands(ins[i])[2], "a")
    for line in ins[mf[0]:mf[-1]]:
        if line.startswith("v_mfma") or not _operands(line):
            continue
        if line.startswith(("s_", "ds_write", "global_store", "buffer_store")):
            continue  # no AGPR destination
        if _regs(_operands(line)[0], "a") & b_regs:
            raise RuntimeError(f"{kernel}: {line!r} writes a query AGPR between the QK MFMAs")


def check_asm_mfma_result_reads(text, kernel):
    """The QK MFMAs of the small-row kernel are asm statements (B operand in
    AGPRs) whose VGPR results the compiler does not know to be late:
    require that no VALU or LDS-write instruction reads one of their results
    before the next drain (an 's_nop 7'). Later MFMAs may read it (as their
    accumulator: the matrix unit orders that itself)."""
    ins = _kernel_body(text, kernel)
    for i, line in enumerate(ins):
        if not (line.startswith("v_mfma") and ", a[" in line):
            continue
        dst = _vregs(line.split(None, 1)[1].split(",")[0].strip())
        for later in ins[i + 1:i + 400]:
            if later.startswith("s_nop 7"):
                break
            if later.startswith("v_mfma"):
                continue
            if (later.startswith("v_") or later.startswith("ds_write")) and "," in later:
                srcs = set()
                for tok in later.split(None, 1)[1].split(",")[1:]:
                    srcs |= _vregs(tok.strip())
                if srcs & dst:
                    raise RuntimeError(f"{kernel}: {later!r} reads the result of {line!r} before a drain")


def build(out: str = LIB, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    check_registers(extra)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
