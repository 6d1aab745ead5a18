"""Host-sanitizer build of liblmhead.so, for the CPU tests.

    python -m vocab_shortlisted_lm_amd.build_sanitized [-o PATH]

The library's host code (argument checks, launch planning, the C ABI) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer; the device
pass is the normal one (same flags, same kernels, the same resource-usage
remarks), so one compile serves both the sanitizer tests and the build's
register and scratch checks.  Load it with LMHEAD_LIB=<path> and the ASan
runtime preloaded (asan_runtime()).
"""
from __future__ import annotations

import argparse
import os
import subprocess

from . import build as _build
from .build import hipcc

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "liblmhead_hostsan.so")


def command(out: str = OUT) -> list[str]:
    """The library's own build command with the sanitizers added to the host
    pass only (each -fsanitize= behind -Xarch_host)."""
    cmd = _build.command(out)
    extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g", "-shared-libsan"]
    return cmd[:-3] + extra + cmd[-3:]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload into Python)."""
    clang = os.path.join(os.path.dirname(hipcc()), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def build(out: str = OUT) -> tuple[str, dict]:
    """Compile; returns (path, per-kernel resource usage from the device
    pass's remarks, as vocab_shortlisted_lm_amd.build.kernel_resources)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    proc = subprocess.run(command(out), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(command(out)) + "\n" + proc.stderr[-4000:])
    return out, _build.kernel_resources(proc.stderr)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("-o", dest="out", default=OUT)
    print(build(ap.parse_args().out)[0])


if __name__ == "__main__":
    main()
