"""The boundary from C: tests/c_consumer/lmhead_consumer owns its device
buffers, gathers a shortlist (lmhead_trim) and runs the argmax over the
trimmed head with d2t and over the full head without it
(draft_project_argmax), the first as single launches on a state it zeroes
once (draft_project_argmax_fused) and the second without a workspace
(draft_project_argmax_noalloc), with no Python or torch in the process.
Its outputs are checked against the fp64 oracle with the parity rule, and
the single-launch and no-workspace outputs against the ordinary calls bit
for bit."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from parity import check
from test_gpu_parity import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def consumer():
    from vocab_shortlisted_lm_amd import build
    if not os.path.exists(build.CONSUMER):
        build.build_consumer()   # a gcc line, no GPU work
    return build.CONSUMER


@pytest.mark.parametrize("m", [1, 3, 24])
def test_c_program_matches_the_oracle(consumer, tmp_path, m):
    inp = synth.make_config(1)             # 4,096 x 256 head, 512-id list
    w, ids = inp["W"], inp["ids"].astype(np.int32)
    n, k = w.shape
    h = synth.hidden(inp["config"].h_seed[0], 50 + m, m, k)
    files = {name: tmp_path / f"{name}.bin" for name in ("w", "ids", "h", "out")}
    np.ascontiguousarray(w, dtype=np.uint16).tofile(files["w"])
    ids.tofile(files["ids"])
    np.ascontiguousarray(h, dtype=np.uint16).tofile(files["h"])
    log(f"[c consumer] M={m} N={n} K={k} S={ids.size}")
    proc = subprocess.run([consumer, str(n), str(k), str(ids.size), str(m), str(files["w"]), str(files["ids"]),
                           str(files["h"]), str(files["out"])], capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stderr
    assert "ok" in proc.stdout
    out = np.fromfile(files["out"], dtype=np.dtype([("id", "<i4"), ("logit", "<f4")]))
    assert out.size == 4 * m
    trimmed, full, fused, noalloc = out[:m], out[m:2 * m], out[2 * m:3 * m], out[3 * m:]
    check(h, oracle.oracle_trim(w, ids), ids, trimmed["id"], trimmed["logit"])
    check(h, w, None, full["id"], full["logit"])
    assert np.array_equal(fused.view(np.uint64), trimmed.view(np.uint64))
    assert np.array_equal(noalloc.view(np.uint64), full.view(np.uint64))
