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
    need = {"verify_attn_partial_kernel": lambda n: n == 256,
            "verify_attn_f32_partial_kernel": lambda n: n >= 128}
    for kname, agpr_ok in need.items():
        found = [v for k, v in info.items() if kname + "E" in k]
        if len(found) != 1:
            raise RuntimeError(f"{kname} not found in the assembly metadata: {sorted(info)}")
        p = found[0]
        if p["vgpr_spill"] or p["sgpr_spill"] or not agpr_ok(p["agpr"]):
            raise RuntimeError(f"{kname} register allocation changed: {p}")
    return info


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
