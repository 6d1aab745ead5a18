"""bench.py's host-side logic, without a GPU: the one-GPU refusal, the
algorithmic byte counts behind roofline.achieved, the digest that ties
committed HBM counters to the kernel code, and the counter bookkeeping
(scaling by the copy kernel, lookup, staleness)."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

K, N = 2560, 248_320


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    p = run_bench("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


@pytest.mark.parametrize("args, text", [
    (("--topk", "4", "--logits", "rows"), "exclude each other"),
    (("--topk", "17"), "--topk must be"),
    (("--fp8", "--mxfp4"), "exclude each other"),
    (("--config", "2", "--indexed"), "--indexed needs a shortlist config"),
    (("--logits", "rows", "--fp8"), "bf16 head"),
])
def test_conflicting_options_exit_before_any_gpu_work(args, text):
    p = run_bench(*args)
    assert p.returncode != 0
    assert text in (p.stderr + p.stdout)


def test_algorithmic_bytes_of_the_full_head():
    # bf16: every weight row once (K x 2 bytes) plus the hidden row
    assert bench.projection_bytes(1, N, K) == N * K * 2 + K * 2 == 1_271_403_520
    # the whole call adds the two outputs (4 + 4 bytes per hidden row) and,
    # with a d2t table, the 4-byte entry of each winner
    assert bench.algorithmic_bytes(1, N, K, with_d2t=False) == 1_271_403_520 + 8
    assert bench.algorithmic_bytes(24, 52_755, K, with_d2t=True) == 52_755 * K * 2 + 24 * K * 2 + 24 * 12
    # FP8: one byte per weight and one fp32 scale per row
    assert bench.projection_bytes(1, N, K, "fp8") == N * K + N * 4 + K * 2 == 636_697_600
    # MXFP4: two codes per byte and one scale byte per 32 weights (1,360 B per row)
    assert bench.head_bytes(1, K, "mxfp4") == 1_360
    assert bench.projection_bytes(1, N, K, "mxfp4") == 337_720_320
    # rows read in place through the list: 4 more bytes per list entry
    assert bench.projection_bytes(3, 16_000, K, indexed=True) == 16_000 * (K * 2 + 4) + 3 * K * 2


def test_digest_ignores_comments_and_whitespace_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"

    def digest(text):
        src.write_text(text)
        monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
        return bench.source_digest()

    base = digest('int f(int x) { return x + 1; }  // one\nconst char* s = "a // b";\n')
    assert digest('/* two */ int f(int x)   {\n  return x + 1;\n}\nconst char* s = "a // b"; // three\n') == base
    assert digest('int f(int x) { return x + 2; }\nconst char* s = "a // b";\n') != base
    # text inside a string literal is code, even when it looks like a comment
    assert digest('int f(int x) { return x + 1; }\nconst char* s = "a // c";\n') != base


def test_committed_counters_are_consistent_and_never_stale():
    """profiles/traffic.json: an entry taken on the kernel code as it stands
    is reported by the benchmark line and shows the head read once: at most
    2% above the algorithmic bytes, beyond the hidden rows fetched once more
    by each further chiplet's L2 (7 x M x K x 2 bytes) and one 32-byte write
    per key slot (M x 1,024 x 32 bytes at most).  A second read of the head
    would add 100%.  An entry taken on other kernel code is never reported
    (the line's `traffic` is then null, not an old figure)."""
    with open(bench.TRAFFIC_FILE) as f:
        table = json.load(f)
    assert table["entries"], "no counter entries"
    digest = bench.source_digest()
    for e in table["entries"]:
        alg = e["algorithmic_bytes_projection_kernel"]
        m = int(re.search(r"M=(\d+)", e["workload"]).group(1))
        k = int(re.search(r"K=(\d+)", e["workload"]).group(1))
        allowance = 7 * m * k * 2 + m * 1024 * 32
        assert e["bytes_projection_kernel"] >= alg, e["workload"]
        if e["source_sha256_16"] == digest:
            assert e["bytes_projection_kernel"] < 1.02 * alg + allowance, e["workload"]
            assert bench.measured_traffic(e["path"], e["workload"]) == e["bytes_projection_kernel"]
        else:
            assert bench.measured_traffic(e["path"], e["workload"]) is None, e["workload"]


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_record_and_look_up_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kern = "void (anonymous namespace)::proj_valu_tiled<1, 4, 4, 1, false, 1>(unsigned short const*)"
    fold = "(anonymous namespace)::finalize_argmax(unsigned long long const*, int)"
    gib_kib = (1 << 30) / 1024
    # the fetch counter reads half the bytes (as on MI355X), the write counter all of them
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(kern, 100.0), (kern, 110.0), (kern, 120.0), (fold, 2.0), ("copy16(int)", gib_kib / 2)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(kern, 8.0), (kern, 8.0), (fold, 0.5), ("copy16(int)", gib_kib)])

    class A:
        indexed = False

    class C:
        k = K

    d = {"kname": "proj_valu_tiled", "kpath": "valu", "workload": "w1", "m": 1, "rows": N, "c": C, "fmt": "bf16"}
    assert bench.record_traffic(A, d, str(tmp_path / "f.csv"), str(tmp_path / "w.csv")) == 0
    e = json.load(open(tmp_path / "traffic.json"))["entries"][0]
    assert e["fetch_kib_per_dispatch"] == 110.0           # the median dispatch
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["bytes_projection_kernel"] == 110 * 1024 * 2 + 8 * 1024
    assert e["algorithmic_bytes_projection_kernel"] == 1_271_403_520
    assert bench.measured_traffic("valu", "w1") == e["bytes_projection_kernel"]
    assert bench.measured_traffic("valu", "w2") is None
    # counters taken on other kernel code are not reported
    src = tmp_path / "k.hip"
    src.write_text("int changed;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    assert bench.measured_traffic("valu", "w1") is None


def test_cpu_baseline_names_its_cores_and_blas():
    """The CPU baseline record states the threads the oracle ran on, the
    host's CPU count and the BLAS library, each as its own field, and the
    time per call and effective rate over the head's bytes."""
    import numpy as np
    import synth
    inp = synth.make_config(1)
    h = synth.hidden(101, 0, 1, 256)
    rec = bench.cpu_baseline(h, inp["W"], None, 0.05)
    assert rec["kind"] == "oracle" and rec["unit"] == "calls/s" and rec["value"] > 0
    assert rec["host_cpus"] == os.cpu_count()
    assert 1 <= rec["host_cpus_usable"] <= os.cpu_count()
    assert rec["cores"] == rec["blas_threads"] >= 1
    assert rec["blas"] != "unknown" and rec["blas"] in rec["sample"]
    assert np.isfinite(rec["value"])
    # seconds per call and the bf16 head bytes it reads per second
    assert abs(rec["seconds_per_call"] * rec["value"] - 1.0) < 1e-9
    assert abs(rec["gbps"] - 4096 * 256 * 2 * rec["value"] / 1e9) <= 1e-3


def test_traffic_table_lists_every_entry():
    """`bench.py --traffic-table` (no GPU) prints one markdown row per entry
    of profiles/traffic.json, with its excess over the algorithmic bytes."""
    with open(bench.TRAFFIC_FILE) as f:
        entries = json.load(f)["entries"]
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-table"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    rows = [ln for ln in p.stdout.splitlines() if ln.startswith("| ") and "`" in ln]
    assert len(rows) == len(entries)
    for e, ln in zip(entries, rows):
        assert e["workload"] in ln and f"{e['bytes_projection_kernel']:,}" in ln


def test_kernel_name_follows_the_library_plan():
    """The kernel whose counters and times a bench line reports: the tiled
    VALU kernel at one and two hidden rows over a head or trimmed list, the
    row-order kernel from three rows and for rows read in place."""
    assert bench.kernel_name("valu", 1) == "proj_valu_tiled"
    assert bench.kernel_name("valu", 2) == "proj_valu_tiled"
    assert bench.kernel_name("valu", 1, True) == "proj_valu_rows"
    assert bench.kernel_name("valu", 2, True) == "proj_valu_rows"
    assert bench.kernel_name("valu", 3) == "proj_valu_rows"
    assert bench.kernel_name("mfma", 1) == "proj_mfma"
