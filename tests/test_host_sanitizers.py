"""The library's build, checked on the CPU from one compile: the library's
own build command with AddressSanitizer and UndefinedBehaviorSanitizer added
to the host pass only.  The device pass is the normal one, so its
resource-usage remarks are the shipped kernels': no kernel spills to scratch
memory, and the one-tile matrix-core argmax kernels fit 4 waves per SIMD.
Then the host-side tests of the C ABI (argument checks, status strings,
workspace and scale-array sizes, the kernel-choice queries, the binding's
own checks) run against the sanitized library in a child Python with the
ASan runtime preloaded: every call there returns before its first launch,
and a heap or stack overrun, a misaligned or out-of-range access, or an
integer overflow in those paths fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    sys.path.insert(0, ROOT)
    from vocab_shortlisted_lm_amd import build_sanitized
    out = str(tmp_path_factory.mktemp("hostsan") / "liblmhead_hostsan.so")
    lib, usage = build_sanitized.build(out)
    return lib, usage, build_sanitized.asan_runtime()


def test_build_has_no_scratch_spills(sanitized):
    """Every kernel keeps its state in registers and LDS."""
    _, usage, _ = sanitized
    for kernel in ("proj_valu_tiled", "proj_valu_rows", "proj_mfma", "finalize_topk", "proj_valu_fp8",
                   "quantize_rows_fp8", "quantize_rows_mxfp4", "quantize_rows_nvfp4", "tile_block_scales",
                   "finalize_keys"):
        assert any(kernel in k for k in usage), kernel
    spills = {k: v["ScratchSize"] for k, v in usage.items() if v.get("ScratchSize", 0)}
    assert not spills, spills
    # The one-tile matrix-core argmax kernels over FP8, MXFP4 and NVFP4 heads
    # run two 8-wave workgroups per CU at a few hidden rows (their LDS allows
    # it), so they must fit 4 waves per SIMD in registers; a larger register
    # peak silently halves their residency (no parity test can see it)
    for fmt, sb in ((1, 8), (2, 16), (3, 16)):
        name = [k for k in usage if "proj_mfma" in k and f"ILi1ELi{sb}ELi8ELi3ELi1ELb0ELi{fmt}ELb0E" in k]
        assert len(name) == 1, (fmt, name)
        assert usage[name[0]].get("Occupancy", 0) >= 4, (name[0], usage[name[0]])


def test_host_checks_under_asan_and_ubsan(sanitized):
    lib, _, runtime = sanitized
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, LMHEAD_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    select = ("rejects or bound or status_strings or workspace_bytes or auto_path or scale_bytes "
              "or declares or exported or targets")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), "-k", select],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in p.stdout and " failed" not in p.stdout, p.stdout[-2000:]
