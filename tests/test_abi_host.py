"""The C-ABI library loads, exports every symbol include/*.h declares,
and rejects bad arguments on the host before touching the GPU (CPU only:
every call here returns before the first HIP runtime call)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def L():
    from vocab_shortlisted_lm_amd import lmhead, build
    src = build.SRC
    if (not os.path.exists(lmhead.LIB_PATH)
            or os.path.getmtime(lmhead.LIB_PATH) < max(os.path.getmtime(f) for f in [src] + HEADERS)):
        build.build()
    return lmhead


def declared_functions(headers=None):
    names = set()
    for path in headers or HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions([HEADER])
    for n in ("lmhead_trim", "draft_project_argmax", "draft_project_workspace_bytes",
              "lmhead_status_str"):
        assert n in names
    # measurement and forced-kernel calls live in lmhead_bench.h, not in the
    # product header
    assert not [n for n in names if n.startswith("lmhead_bench_")]
    assert "draft_project_argmax_path" not in names
    bench = declared_functions([os.path.join(ROOT, "include", "lmhead_bench.h")])
    assert "draft_project_argmax_path" in bench and "lmhead_bench_time_argmax" in bench


def test_every_declared_symbol_is_exported(L):
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    assert set(L.SIGNATURES) == set(declared_functions())


def test_library_targets_gfx950_only(L):
    data = open(L.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-\w:+]*", data))
    assert targets == {b"amdgcn-amd-amdhsa--gfx950"}, targets


def test_status_strings(L):
    for c in range(5):
        assert L.lmhead_status_str(c)
    assert "range" in L.lmhead_status_str(L.LMH_ERANGE)
    assert L.lmhead_status_str(99) == "unknown status"


def test_workspace_bytes(L):
    assert L.draft_project_workspace_bytes(0) == 0
    assert L.draft_project_workspace_bytes(33) == 0
    for m in (1, 3, 24, 32):
        ws = L.draft_project_workspace_bytes(m)
        assert ws == m * 1024 * 8 and ws % 16 == 0


def test_fused_state_size(L):
    """The single-launch state holds the tickets and keys of 16 merge groups
    and of the final level within LMH_STATE_BYTES."""
    assert L.LMH_STATE_BYTES == 8192
    src = open(os.path.join(ROOT, "include", "lmhead.h")).read()
    assert "#define LMH_STATE_BYTES 8192" in src


def test_auto_path_by_head_size(L):
    # the head's size does not change the choice: VALU up to four hidden
    # rows, matrix cores from five, on lists and on the full head
    assert L.draft_project_auto_path_rows(4, 2560, 32768) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(4, 2560, 131071) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(4, 2560, 131072) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(4, 2560, 248320) == L.LMH_PATH_VALU
    for m in (1, 2, 3):
        assert L.draft_project_auto_path_rows(m, 2560, 16000) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(5, 2560, 248320) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path_rows(5, 2560, 16000) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path_rows(4, 2560, (1 << 30) - 1) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path_rows(4, 2560, 1 << 30) == -1
    assert L.draft_project_auto_path_rows(4, 2560, 0) == -1
    assert L.draft_project_auto_path_rows(0, 2560, 100) == -1


def test_auto_path(L):
    assert L.draft_project_auto_path(1, 2560) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path(4, 2560) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path(3, 2560) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path(5, 2560) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path(8, 2560) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path(9, 2560) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path(24, 2560) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path(4, 8192) == L.LMH_PATH_MFMA
    assert L.draft_project_auto_path(2, 8192) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path(4, 4096) == L.LMH_PATH_VALU
    assert L.draft_project_auto_path(1, 8192) == L.LMH_PATH_VALU
    for m, k in ((0, 2560), (33, 2560), (1, 12), (1, 0), (1, 8200)):
        assert L.draft_project_auto_path(m, k) == -1


# fake, aligned addresses: validation must reject before any device access
A, B, C, D, E = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def call(L, h=A, m=1, k=2560, w=B, r=100, d2t=None, oid=C, olog=D, ws=E, wsb=1 << 20, path=0):
    return L.lib().draft_project_argmax_path(h, m, k, w, r, d2t, oid, olog, ws, wsb, path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), 1), (dict(w=None), 1), (dict(oid=None), 1), (dict(olog=None), 1),
    (dict(m=0), 1), (dict(m=33), 1), (dict(k=0), 1), (dict(k=12), 1), (dict(k=8200), 1),
    (dict(r=0), 1), (dict(r=1 << 30), 1), (dict(r=(1 << 30) + 1), 1), (dict(h=A + 2), 1), (dict(w=B + 8), 1),
    (dict(path=7), 1), (dict(m=9, path=1), 1), (dict(m=4, k=8192, path=1), 1), (dict(m=8, k=4096, path=1), 1),
    (dict(ws=None), 3), (dict(ws=E + 4), 3), (dict(wsb=16), 3), (dict(wsb=0), 3),
    (dict(m=2, wsb=8 * 1024 * 2 - 8), 3),
])
def test_project_rejects_on_host(L, kw, code):
    assert call(L, **kw) == code


def topk_call(L, h=A, m=2, k=2560, w=B, r=100, d2t=None, topk=4, oid=C, olog=D, ws=E,
              wsb=1 << 24, path=0):
    return L.lib().draft_project_topk(h, m, k, w, r, d2t, topk, oid, olog, ws, wsb, path, None)


@pytest.mark.parametrize("kw,code", [
    (dict(topk=0), 1), (dict(topk=17), 1), (dict(oid=None), 1), (dict(olog=None), 1),
    (dict(h=None), 1), (dict(m=0), 1), (dict(k=12), 1), (dict(r=0), 1), (dict(w=B + 2), 1),
    (dict(m=5, path=1), 1), (dict(path=3), 1), (dict(ws=None), 3), (dict(ws=E + 8), 3),
    (dict(wsb=2 * 1024 * 4 * 8 - 1), 3),
])
def test_topk_rejects_on_host(L, kw, code):
    assert topk_call(L, **kw) == code


def test_topk_workspace_bytes(L):
    assert L.draft_project_topk_workspace_bytes(1, 1) == 8 * 1024
    assert L.draft_project_topk_workspace_bytes(2, 3) == 2 * 1024 * 4 * 8
    assert L.draft_project_topk_workspace_bytes(24, 16) == 24 * 1024 * 16 * 8
    assert L.draft_project_topk_workspace_bytes(1, 17) == 0
    assert L.draft_project_topk_workspace_bytes(33, 4) == 0


def test_logits_rejects_on_host(L):
    lib = L.lib()
    f = lib.draft_project_logits
    assert f(A, 1, 2560, B, 100, None, 0, None, 0, None) == 1          # no output
    assert f(A, 1, 2560, B, 100, None, 0, C + 2, 0, None) == 1         # misaligned output
    assert f(A, 1, 2560, B, 100, D, 0, C, 0, None) == 1                # d2t needs N >= 1
    assert f(A, 5, 2560, B, 100, None, 0, C, 1, None) == 1             # VALU epilogues: M <= 4
    assert f(A, 3, 8192, B, 100, None, 0, C, 1, None) == 1             # and M * ceil(K / 512) <= 40
    assert f(A, 1, 12, B, 100, None, 0, C, 0, None) == 1


def test_bench_time_rejects_on_host(L):
    import ctypes
    f = L.lib().lmhead_bench_time_argmax
    one = (ctypes.c_void_p * 1)(B)
    out = ctypes.c_double(0.0)
    ws = L.draft_project_workspace_bytes(1)
    assert f(A, 1, 2560, None, 1, 100, None, C, D, E, ws, 0, 5, ctypes.byref(out), None) == 1  # no heads
    assert f(A, 1, 2560, one, 0, 100, None, C, D, E, ws, 0, 5, ctypes.byref(out), None) == 1   # nheads 0
    assert f(A, 1, 2560, one, 1, 100, None, C, D, E, ws, 0, 0, ctypes.byref(out), None) == 1   # calls 0
    assert f(A, 1, 2560, one, 1, 100, None, C, D, E, ws, 0, 5, None, None) == 1                # no output
    assert f(A, 1, 2560, one, 1, 100, None, C, D, E, 8, 0, 5, ctypes.byref(out), None) == 3    # workspace


def test_fp8_rejects_on_host(L):
    lib = L.lib()
    q = lib.lmhead_quantize_fp8
    assert q(A, 0, 2560, B, C, None) == 0                        # R = 0: no-op
    assert q(A, 10, 2568, B, C, None) == 1                       # K not a multiple of 16
    assert q(A, 10, 2560, B + 8, C, None) == 1                   # Wq misaligned
    assert q(A, 10, 2560, B, C + 2, None) == 1                   # scale misaligned
    assert q(None, 10, 2560, B, C, None) == 1
    assert q(A, -1, 2560, B, C, None) == 1
    f = lib.draft_project_argmax_fp8
    ws = L.draft_project_workspace_bytes(4)
    assert f(A, 4, 2568, B, C, 100, None, D, E, E, ws, 0, None) == 1   # K % 16
    assert f(A, 5, 2560, B, C, 100, None, D, E, E, ws, 1, None) == 1   # VALU takes M <= 4
    assert f(A, 1, 2560, B, None, 100, None, D, E, E, ws, 0, None) == 1  # no scale
    assert f(A, 1, 2560, B, C + 1, 100, None, D, E, E, ws, 0, None) == 1
    assert f(A, 33, 2560, B, C, 100, None, D, E, E, ws, 0, None) == 1
    assert f(A, 1, 2560, B, C, 0, None, D, E, E, ws, 0, None) == 1     # R = 0
    assert f(A, 4, 2560, B, C, 100, None, D, E, E, 8, 0, None) == 3    # workspace


def test_indexed_rejects_on_host(L):
    import ctypes
    f = L.lib().draft_project_argmax_indexed
    ws = L.draft_project_workspace_bytes(3)
    assert f(A, 3, 2560, B, 0, C, 100, D, E, E, ws, 0, None) == 1      # N = 0
    assert f(A, 3, 2560, B, 1 << 31, C, 100, D, E, E, ws, 0, None) == 1  # N >= 2^31
    assert f(A, 3, 2560, B, 1000, None, 100, D, E, E, ws, 0, None) == 1  # no ids
    assert f(A, 3, 2560, B, 1000, C + 2, 100, D, E, E, ws, 0, None) == 1  # ids misaligned
    assert f(A, 3, 2560, B, 1000, C, 0, D, E, E, ws, 0, None) == 1     # S = 0
    assert f(A, 3, 2560, B, 1000, C, (1 << 30) + 1, D, E, E, ws, 0, None) == 1
    assert f(A, 3, 2560, B, 1000, C, 1 << 30, D, E, E, ws, 0, None) == 1  # 4 * S must stay below 2^32
    assert f(A, 33, 2560, B, 1000, C, 100, D, E, E, ws, 0, None) == 1  # M
    assert f(A, 3, 2560, B + 8, 1000, C, 100, D, E, E, ws, 0, None) == 1  # W misaligned
    assert f(A, 9, 2560, B, 1000, C, 100, D, E, E, ws, 1, None) == 1   # VALU takes M <= 8
    assert f(A, 3, 2560, B, 1000, C, 100, None, E, E, ws, 0, None) == 1  # no output
    assert f(A, 3, 2560, B, 1000, C, 100, D, E, E, 8, 0, None) == 3    # workspace
    t = L.lib().lmhead_bench_time_argmax_indexed
    one = (ctypes.c_void_p * 1)(B)
    out = ctypes.c_double(0.0)
    assert t(A, 1, 2560, None, 1, 1000, C, 100, D, E, E, ws, 0, 5, ctypes.byref(out), None) == 1
    assert t(A, 1, 2560, one, 1, 1000, None, 100, D, E, E, ws, 0, 5, ctypes.byref(out), None) == 1
    assert t(A, 1, 2560, one, 1, 1000, C, 100, D, E, E, ws, 0, 0, ctypes.byref(out), None) == 1


def test_mxfp4_scale_bytes_and_tiling_rejects(L):
    lib = L.lib()
    sb = lib.lmhead_mxfp4_scale_bytes
    assert sb(248320, 2560) == 15520 * 5 * 256 == 248320 * 80
    assert sb(1, 32) == 256 and sb(17, 544) == 2 * 2 * 256 and sb(0, 2560) == 0
    assert sb(10, 48) == -1 and sb(-1, 512) == -1 and sb(10, 0) == -1
    assert L.mxfp4_scale_shape(17, 544) == (2, 2, 16, 16)
    t = lib.lmhead_mxfp4_tile_scales
    assert t(A, 0, 2560, B, None) == 0                           # R = 0: no-op
    assert t(A, 10, 48, B, None) == 1
    assert t(None, 10, 512, B, None) == 1
    assert t(A, 10, 512, None, None) == 1
    assert t(A, -3, 512, B, None) == 1


def test_quantized_topk_rejects_on_host(L):
    lib = L.lib()
    ws = L.draft_project_topk_workspace_bytes(4, 8)
    f8, f4 = lib.draft_project_topk_fp8, lib.draft_project_topk_mxfp4
    # FP8: scale pointer 4-byte aligned; K % 16; no VALU path; topk 1-16; workspace
    assert f8(A, 4, 2560, B, C, 100, None, 8, D, E, E, ws, 1, None) == 1
    assert f8(A, 4, 2560, B, C, 100, None, 0, D, E, E, ws, 0, None) == 1
    assert f8(A, 4, 2560, B, C, 100, None, 17, D, E, E, ws, 0, None) == 1
    assert f8(A, 4, 2568, B, C, 100, None, 8, D, E, E, ws, 0, None) == 1
    assert f8(A, 4, 2560, B, C + 2, 100, None, 8, D, E, E, ws, 0, None) == 1
    assert f8(A, 4, 2560, B, C, 100, None, 8, None, E, E, ws, 0, None) == 1
    assert f8(A, 4, 2560, B, C, 100, None, 8, D, E, E, ws - 1, 0, None) == 3
    assert f8(A, 4, 2560, B, C, 100, None, 8, D, E, E + 8, ws, 0, None) == 3
    # MXFP4: K % 512; no VALU path; topk 1-16; workspace
    assert f4(A, 4, 2560, B, C, 100, None, 8, D, E, E, ws, 1, None) == 1
    assert f4(A, 4, 2592, B, C, 100, None, 8, D, E, E, ws, 0, None) == 1
    assert f4(A, 4, 2560, B, C, 100, None, 17, D, E, E, ws, 0, None) == 1
    assert f4(A, 4, 2560, B, C + 4, 100, None, 8, D, E, E, ws, 0, None) == 1
    assert f4(A, 33, 2560, B, C, 100, None, 8, D, E, E, ws, 0, None) == 1
    assert f4(A, 4, 2560, B, C, 100, None, 8, D, E, E, ws - 1, 0, None) == 3


def test_mxfp4_rejects_on_host(L):
    lib = L.lib()
    q = lib.lmhead_quantize_mxfp4
    assert q(A, 0, 2560, B, C, None) == 0                        # R = 0: no-op
    assert q(A, 10, 2576, B, C, None) == 1                       # K not a multiple of 32
    assert q(A, 10, 2560, B + 8, C, None) == 1                   # Wq misaligned
    assert q(None, 10, 2560, B, C, None) == 1
    assert q(A, 10, 2560, B, None, None) == 1
    f = lib.draft_project_argmax_mxfp4
    ws = L.draft_project_workspace_bytes(4)
    assert f(A, 4, 2592, B, C, 100, None, D, E, E, ws, 0, None) == 1   # K % 512
    assert f(A, 4, 2560, B, C, 100, None, D, E, E, ws, 1, None) == 1   # no VALU path
    assert f(A, 4, 2560, B, C + 4, 100, None, D, E, E, ws, 0, None) == 1  # scales misaligned
    assert f(A, 4, 2560, B, None, 100, None, D, E, E, ws, 0, None) == 1
    assert f(A, 33, 2560, B, C, 100, None, D, E, E, ws, 0, None) == 1
    assert f(A, 1, 2560, B, C, 0, None, D, E, E, ws, 0, None) == 1     # R = 0
    assert f(A, 4, 2560, B, C, 100, None, D, E, E, 8, 0, None) == 3    # workspace


def test_nvfp4_rejects_on_host(L):
    lib = L.lib()
    q = lib.lmhead_quantize_nvfp4
    assert q(A, 0, 2560, B, C, D, None) == 0                      # R = 0: no-op
    assert q(A, 10, 2568, B, C, D, None) == 1                     # K not a multiple of 16
    assert q(A, 10, 2560, B + 8, C, D, None) == 1                 # Wq misaligned
    assert q(A, 10, 2560, B, C, D + 2, None) == 1                 # gscale misaligned
    assert q(A, 10, 2560, B, C, None, None) == 1
    assert q(None, 10, 2560, B, C, D, None) == 1
    assert q(A, 1 << 30, 2560, B, C, D, None) == 1
    f = lib.draft_project_argmax_nvfp4
    ws = L.draft_project_workspace_bytes(4)
    assert f(A, 4, 2592, B, C, D, 100, None, E, E, E, ws, 0, None) == 1   # K % 512
    assert f(A, 4, 2560, B, C, D, 100, None, E, E, E, ws, 1, None) == 1   # no VALU path
    assert f(A, 4, 2560, B, C + 4, D, 100, None, E, E, E, ws, 0, None) == 1  # scales misaligned
    assert f(A, 4, 2560, B, C, None, 100, None, E, E, E, ws, 0, None) == 1   # no head scale
    assert f(A, 4, 2560, B, C, D + 1, 100, None, E, E, E, ws, 0, None) == 1  # head scale misaligned
    assert f(A, 33, 2560, B, C, D, 100, None, E, E, E, ws, 0, None) == 1
    assert f(A, 1, 2560, B, C, D, 0, None, E, E, E, ws, 0, None) == 1     # R = 0
    assert f(A, 4, 2560, B, C, D, 100, None, E, E, E, 8, 0, None) == 3    # workspace
    t = lib.draft_project_topk_nvfp4
    assert t(A, 2, 2560, B, C, D, 100, None, 0, E, E, E, 1 << 24, 0, None) == 1   # topk 0
    assert t(A, 2, 2560, B, C, D, 100, None, 4, E, E, E, 1 << 24, 1, None) == 1   # no VALU path
    assert L.lmhead_nvfp4_scale_bytes(17, 2560) == 2 * 5 * 512
    assert L.lmhead_nvfp4_scale_bytes(16, 16) == 512
    assert L.lmhead_nvfp4_scale_bytes(16, 24) == -1
    assert L.nvfp4_scale_shape(17, 2560) == (2, 5, 16, 32)
    tl = lib.lmhead_nvfp4_tile_scales
    assert tl(A, 0, 2560, B, None) == 0
    assert tl(A, 10, 2568, B, None) == 1
    assert tl(None, 10, 2560, B, None) == 1


def test_shortlist_ops_reject_on_host(L):
    lib = L.lib()
    f = lib.lmhead_shortlist_overwrite
    assert f(A, 100, 256, B, C, 50, D, E, 0, None) == 0                 # n = 0: no-op
    assert f(A, 100, 256, B, C, 50, D, E, 65537, None) == 1             # n > LMH_MAX_OVERWRITE
    assert f(A, 0, 256, B, C, 50, D, E, 4, None) == 1                   # N = 0
    assert f(A, 100, 12, B, C, 50, D, E, 4, None) == 1                  # K
    assert f(A, 100, 256, B, C, 0, D, E, 4, None) == 1                  # cap = 0
    assert f(A, 100, 256, A + 512, C, 50, D, E, 4, None) == 1           # W_trim overlaps W
    assert f(A, 100, 256, B + 8, C, 50, D, E, 4, None) == 1             # misaligned W_trim
    assert f(A, 100, 256, B, None, 50, D, E, 4, None) == 1
    assert f(A, 100, 256, B, C, 50, None, E, 4, None) == 1
    u = lib.lmhead_shortlist_union
    assert u(A, 10, B, 10, 1 << 19 | 1, C, 20, D, None) == 1            # N > LMH_MAX_UNION_VOCAB
    assert u(A, 10, B, 10, 0, C, 20, D, None) == 1
    assert u(A, 10, B, 10, 100, C, 19, D, None) == 1                    # out too small
    assert u(A, 10, B, 10, 100, C, 20, None, None) == 1                 # no counts
    assert u(None, 10, B, 10, 100, C, 20, D, None) == 1
    assert u(A, -1, B, 10, 100, C, 20, D, None) == 1


def test_trim_rejects_on_host(L):
    lib = L.lib()
    assert lib.lmhead_trim(A, 100, 2560, B, 0, C, None) == 0          # S = 0: no-op
    assert lib.lmhead_trim(A, 100, 2560, B, -1, C, None) == 1
    assert lib.lmhead_trim(A, 0, 2560, B, 4, C, None) == 1
    assert lib.lmhead_trim(A, 100, 12, B, 4, C, None) == 1
    assert lib.lmhead_trim(None, 100, 2560, B, 4, C, None) == 1
    assert lib.lmhead_trim(A, 100, 2560, None, 4, C, None) == 1
    assert lib.lmhead_trim(A, 100, 2560, B, 4, None, None) == 1
    assert lib.lmhead_trim(A + 2, 100, 2560, B, 4, C, None) == 1
    assert lib.lmhead_trim(A, 100, 2560, B, 4, C + 8, None) == 1


def test_bench_kernels_reject_on_host(L):
    lib = L.lib()
    assert lib.lmhead_bench_stream_read(A, 1000, B, 0, None) == 1     # not a multiple of 16
    assert lib.lmhead_bench_stream_read(None, 1024, B, 0, None) == 1
    assert lib.lmhead_bench_stream_read(A, 0, B, 0, None) == 1        # nothing to read
    assert lib.lmhead_bench_copy(A, B + 4, 1024, 0, None) == 1
    assert lib.lmhead_bench_sink_words() >= 4096


def test_binding_rejects_host_tensors_before_any_call(L):
    """Every wrapper refuses host tensors before the library sees a pointer
    (a host address in a kernel would fault the GPU)."""
    import torch
    h = torch.zeros(2, 512, dtype=torch.bfloat16)
    W = torch.zeros(64, 512, dtype=torch.bfloat16)
    ids = torch.zeros(4, dtype=torch.int32)
    calls = [
        lambda: L.draft_project_argmax(h, W),
        lambda: L.PreparedArgmax(h, W),
        lambda: L.draft_project_topk(h, W, None, 4),
        lambda: L.draft_project_logits(h, W),
        lambda: L.lmhead_trim(W, ids),
        lambda: L.lmhead_quantize_fp8(W),
        lambda: L.lmhead_quantize_mxfp4(W),
        lambda: L.draft_project_argmax_indexed(h, W, ids),
        lambda: L.lmhead_shortlist_union(ids, ids, 100),
        lambda: L.lmhead_bench_stream_read(W, ids),
        lambda: L.lmhead_bench_copy(W, W),
        lambda: L.lmhead_mxfp4_tile_scales(torch.zeros(64, 16, dtype=torch.uint8)),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError, match="device tensor"):
            call()


def test_read_id_list(L, tmp_path):
    p = tmp_path / "ranks.txt"
    p.write_text("17\n3\n\n248319\n0\n")
    ids = L.read_id_list(str(p))
    assert ids.dtype.name == "int32" and ids.tolist() == [17, 3, 248319, 0]


def test_header_is_plain_c(tmp_path):
    """include/lmhead.h and lmhead_bench.h compile as strict C99 on their own:
    the boundary has no C++ or torch types."""
    src = tmp_path / "uses_header.c"
    src.write_text('#include "lmhead.h"\n#include "lmhead_bench.h"\n'
                   'int main(void) { return (int)draft_project_workspace_bytes(1) == 0; }\n')
    proc = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                           "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr


def test_c_consumer_builds_against_the_header_alone(tmp_path):
    """The C program the boundary test drives (tests/c_consumer) builds with
    gcc from the header and HIP's C runtime API, and resolves the in-tree
    library by a path relative to itself."""
    from vocab_shortlisted_lm_amd import build
    out = build.build_consumer(str(tmp_path / "consumer"))
    ldd = subprocess.run(["ldd", out], capture_output=True, text=True, check=True).stdout
    line = [l for l in ldd.splitlines() if "liblmhead.so" in l]
    assert line and "not found" not in line[0], ldd


def test_row_bound_is_below_two_to_the_thirty(L):
    """Heads and lists are capped at 2^30 - 1 rows on the host, before any
    launch: the id list of an indexed call is read through a buffer
    descriptor whose 32-bit byte count, 4 bytes per entry, would wrap to 0 at
    2^30 entries and make every id read as 0 (a valid row, so a silently
    wrong answer).  Every entry point that takes a row count rejects 2^30."""
    lib = L.lib()
    big = 1 << 30
    assert L.LMH_MAX_R == big - 1
    ws = L.draft_project_workspace_bytes(3)
    assert lib.draft_project_argmax(A, 3, 2560, B, big, None, C, D, E, ws, None) == 1
    assert lib.draft_project_argmax_indexed(A, 3, 2560, B, 1000, C, big, D, E, E, ws, 0, None) == 1
    assert lib.draft_project_topk(A, 2, 2560, B, big, None, 4, C, D, E, 1 << 24, 0, None) == 1
    assert lib.draft_project_logits(A, 1, 2560, B, big, None, 0, D, 0, None) == 1
    assert lib.draft_project_argmax_fp8(A, 1, 2560, B, E, big, None, C, D, E, ws, 0, None) == 1
    assert lib.draft_project_argmax_mxfp4(A, 1, 2560, B, E, big, None, C, D, E, ws, 0, None) == 1
    assert lib.lmhead_quantize_fp8(A, big, 2560, B, E, None) == 1
    assert lib.lmhead_quantize_mxfp4(A, big, 2560, B, E, None) == 1
    assert lib.lmhead_mxfp4_scale_bytes(big, 2560) == -1
    assert lib.lmhead_mxfp4_scale_bytes(big - 1, 2560) == (big // 16) * 5 * 256
    assert lib.draft_project_auto_path_rows(1, 2560, big) == -1
    assert lib.draft_project_auto_path_rows(1, 2560, big - 1) in (1, 2)


def test_noalloc_rejects_on_host(L):
    """The allocation-free argmax checks its arguments before it looks up
    its scratch array or launches anything."""
    f = L.lib().draft_project_argmax_noalloc
    assert L.LMH_NOALLOC_MAX_M == L.LMH_MAX_M
    assert f(A, 33, 2560, B, 100, None, C, D, None) == 1          # M above the array's rows
    assert f(A, 0, 2560, B, 100, None, C, D, None) == 1
    assert f(A, 2, 2560, B, 0, None, C, D, None) == 1             # R = 0
    assert f(A, 2, 2560, B, 1 << 30, None, C, D, None) == 1
    assert f(A, 2, 2564, B, 100, None, C, D, None) == 1           # K % 8
    assert f(A + 2, 2, 2560, B, 100, None, C, D, None) == 1       # h misaligned
    assert f(A, 2, 2560, B, 100, None, None, D, None) == 1
    assert f(A, 2, 2560, B, 100, None, C, None, None) == 1


def test_fused_rejects_on_host(L):
    """The single-launch argmax checks its arguments, the state included,
    before anything is launched."""
    f = L.lib().draft_project_argmax_fused
    g = L.lib().draft_project_argmax_fused_path
    S = L.LMH_STATE_BYTES
    assert f(A, 2, 2560, B, 100, None, C, D, None, S, None) == 3          # no state
    assert f(A, 2, 2560, B, 100, None, C, D, E + 8, S, None) == 3         # misaligned state
    assert f(A, 2, 2560, B, 100, None, C, D, E, S - 1, None) == 3         # state too small
    assert f(A, 33, 2560, B, 100, None, C, D, E, S, None) == 1
    assert f(A, 2, 2560, B, 0, None, C, D, E, S, None) == 1
    assert f(A, 2, 2560, B, 1 << 30, None, C, D, E, S, None) == 1
    assert f(A, 2, 2564, B, 100, None, C, D, E, S, None) == 1
    assert f(A, 2, 2560, B, 100, None, None, D, E, S, None) == 1
    assert f(A, 2, 2560, B, 100, None, C, None, E, S, None) == 1
    assert g(A, 2, 2560, B, 100, None, C, D, E, S, 3, None) == 1          # no such path
    assert g(A, 9, 2560, B, 100, None, C, D, E, S, L.LMH_PATH_VALU, None) == 1   # VALU argmax: M <= 8
