"""Build liblmhead.so (HIP, gfx950) in-tree with hipcc.

    python -m vocab_shortlisted_lm_amd.build [-D NAME=VALUE ...] [-o PATH]

The library is one translation unit, csrc/lmhead.hip, compiled for gfx950
only.  Packed-fp32 instruction selection is switched off on the device pass
(`-target-feature -packed-fp32-ops`); the host pass prints a harmless warning
that it does not know that feature.
"""
from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "lmhead.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblmhead.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def command(out: str = LIB, defines: list[str] | None = None) -> list[str]:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE]
    for d in defines or []:
        cmd.append("-D" + d)
    cmd += [SRC, "-o", out]
    return cmd


def kernel_resources(stderr: str) -> dict[str, dict[str, int]]:
    """Per-kernel resource usage from the compiler's kernel-resource-usage
    remarks: {mangled name: {"ScratchSize": bytes/lane, "VGPRs": n, ...}}."""
    usage: dict[str, dict[str, int]] = {}
    name = None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(\w+)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            usage[name][m.group(1)] = int(m.group(2))
    return usage


def build(out: str = LIB, defines: list[str] | None = None, verbose: bool = False,
          allow_scratch: bool = False) -> str:
    """Compile the library; returns its path.  Raises on a compiler error,
    and -- unless allow_scratch -- if any kernel spills to scratch memory
    (a spill in a streaming kernel costs far more than the register it saves)."""
    tmp = out + ".tmp"
    cmd = command(tmp, defines)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in proc.stderr.splitlines() if noise not in l]
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    spills = {k: v["ScratchSize"] for k, v in kernel_resources(proc.stderr).items()
              if v.get("ScratchSize", 0) > 0}
    if spills and not allow_scratch:
        os.remove(tmp)
        raise RuntimeError("kernels spill to scratch: " + ", ".join(f"{k} ({v} B/lane)"
                                                                   for k, v in spills.items()))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


CONSUMER_SRC = os.path.join(ROOT, "tests", "c_consumer", "lmhead_consumer.c")
CONSUMER = os.path.join(ROOT, "tests", "c_consumer", "lmhead_consumer")


def build_consumer(out: str = CONSUMER) -> str:
    """Compile the C program that drives the library through the header
    alone (C11, gcc, HIP's C runtime API), linked against the in-tree
    library by a path relative to the program."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rel = os.path.relpath(PKG, os.path.dirname(out))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, CONSUMER_SRC, "-o", out,
           "-L", PKG, "-llmhead", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("gcc failed:\n" + " ".join(cmd) + "\n" + proc.stderr)
    return out


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("-o", dest="out", default=LIB)
    ap.add_argument("--allow-scratch", action="store_true")
    a = ap.parse_args()
    print(build(a.out, a.defines, verbose=True, allow_scratch=a.allow_scratch))


if __name__ == "__main__":
    main()
