#!/usr/bin/env python3
"""Draft-head projection benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2] [--path auto|valu|mfma]

A step is one draft_project_argmax call (projection + fused argmax + d2t map)
over one hidden block, with every input already resident in HBM.  The
default workload is the full-vocabulary draft step: M = 1 hidden row of
width K = 2,560 against all N = 248,320 rows of a bf16 LM head (synthetic,
seeded).  Prints ONE JSON line with calls/s over the timed steps, the
projection kernel's achieved algorithmic HBM bandwidth against the 8 TB/s
MI355X peak (its mean duration from two HIP events the library records
around as many projection launches again, back to back on the same stream,
right after the timed region), and the fp64 CPU oracle timed on a bounded
sample of the same workload.

Other configs (--config 1, 3, 4, 5) are for exploration; shortlist configs
rotate through enough W_trim copies to exceed the 256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "draft-head calls/sec + achieved HBM GB/s (% of peak), M=1 K=2560 N=248,320"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20      # Infinity Cache
KERNEL_SOURCE = os.path.join(ROOT, "vocab_shortlisted_lm_amd", "csrc", "lmhead.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def weight_bytes(rows: int, k: int) -> int:
    """bf16 weight bytes streamed by one projection over `rows` head rows."""
    return rows * k * 2


def algorithmic_bytes(m: int, rows: int, k: int, with_d2t: bool, fmt: str = "bf16",
                      indexed: bool = False) -> int:
    """Bytes one whole call must move at least: every weight row once, the
    hidden rows once, the d2t entries of the winners and the two outputs."""
    return projection_bytes(m, rows, k, fmt, indexed) + (4 * m if with_d2t else 0) + 8 * m


def head_bytes(rows: int, k: int, fmt: str = "bf16") -> int:
    """Bytes of the head: bf16; E4M3 codes plus one fp32 scale per row;
    MXFP4 codes (two per byte) plus one E8M0 scale byte per 32 elements; or
    NVFP4 codes plus one E4M3 scale byte per 16 elements and the head's fp32
    scale."""
    if fmt == "fp8":
        return rows * k + rows * 4
    if fmt == "mxfp4":
        return rows * (k // 2) + rows * (k // 32)
    if fmt == "nvfp4":
        return rows * (k // 2) + rows * (k // 16) + 4
    return weight_bytes(rows, k)


def projection_bytes(m: int, rows: int, k: int, fmt: str = "bf16", indexed: bool = False) -> int:
    """Bytes the projection kernel itself must move: every weight row once
    (in the head's format), the id list when the rows are read in place from
    the full head (4 bytes per entry), and the hidden rows once (the fold and
    the d2t map run afterwards)."""
    return head_bytes(rows, k, fmt) + (rows * 4 if indexed else 0) + m * k * 2


_CODE_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def source_digest() -> str:
    """Digest of the kernel source's code: comments dropped, string and
    character literals kept, runs of whitespace folded, so that counters
    taken on a kernel stay valid across edits of its comments only."""
    with open(KERNEL_SOURCE, encoding="utf-8") as f:
        text = f.read()
    code = _CODE_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def kernel_name(path: str, m: int, indexed: bool = False) -> str:
    """The projection kernel a call runs (the plan in the library's host code:
    the tiled kernel at one and two hidden rows, except over rows read in
    place through a list, which take the row-order kernel)."""
    if path == "mfma":
        return "proj_mfma"
    return "proj_valu_tiled" if m <= 2 and not indexed else "proj_valu_rows"


def describe(a, synth, L):
    """Everything about the workload that needs no GPU."""
    inp = synth.make_config(a.config)
    c = inp["config"]
    m = a.m if a.m is not None else c.ms[0]
    ids = inp["ids"]
    trimmed = ids is not None and not a.full
    path = {"auto": L.LMH_PATH_AUTO, "valu": L.LMH_PATH_VALU, "mfma": L.LMH_PATH_MFMA}[a.path]
    quantized = a.fp8 or a.mxfp4 or a.nvfp4
    if quantized:
        chosen = L.LMH_PATH_MFMA if path == L.LMH_PATH_AUTO else path   # the library's quantized-head default
    else:
        rows_now = c.n if (ids is None or a.full) else ids.size
        # the library's choice: by head size for an argmax over a trimmed or
        # full head; indexed, top-k and logits calls keep the full-head rule
        by_rows = not (a.indexed or a.topk or a.logits)
        chosen = (path if path != L.LMH_PATH_AUTO else
                  L.draft_project_auto_path_rows(m, c.k, rows_now) if by_rows else L.draft_project_auto_path(m, c.k))
    if a.rows:
        if ids is not None and not a.full:
            raise SystemExit("bench.py: --rows slices the full head: use --config 2, or --full")
        if quantized or a.indexed or a.topk or a.logits or a.fused:
            raise SystemExit("bench.py: --rows times the bf16 argmax keys of a head slice")
        if not 1 <= a.rows <= c.n:
            raise SystemExit(f"bench.py: --rows must be 1..{c.n}")
        chosen = path if path != L.LMH_PATH_AUTO else L.draft_project_auto_path_rows(m, c.k, a.rows)
    kpath = {L.LMH_PATH_VALU: "valu", L.LMH_PATH_MFMA: "mfma"}[chosen]
    if a.rows:
        rows = a.rows
        copies = max(1, -(-2 * MALL_BYTES // weight_bytes(rows, c.k)) + 1) if weight_bytes(rows, c.k) < 2 * MALL_BYTES \
            else 1
        workload = (f"vocab shard: M={m} K={c.k} rows 0..{rows - 1} of the N={c.n} head, argmax keys "
                    f"({copies} rotated copies)")
        trimmed = False
        ids = None
    elif trimmed:
        rows = ids.size
        copies = max(1, -(-2 * MALL_BYTES // weight_bytes(rows, c.k)) + 1)
        workload = f"{c.name}: M={m} K={c.k} trimmed to {rows} rows ({copies} rotated copies)"
    else:
        rows, copies = c.n, 1
        workload = (f"full-vocab draft step M={m} K={c.k} N={c.n}" if a.config == 2
                    else f"{c.name}: M={m} K={c.k} full head N={c.n}")
    if (a.fp8 + a.mxfp4 + a.nvfp4) > 1:
        raise SystemExit("bench.py: --fp8, --mxfp4 and --nvfp4 exclude each other")
    if a.topk and a.logits:
        raise SystemExit("bench.py: --topk and --logits exclude each other")
    if (a.topk or a.logits) and a.indexed:
        raise SystemExit("bench.py: --topk and --logits time trimmed or full heads, not --indexed")
    if a.logits and quantized:
        raise SystemExit("bench.py: --logits takes a bf16 head")
    if a.fused and (quantized or a.indexed or a.topk or a.logits):
        raise SystemExit("bench.py: --fused times the bf16 argmax over a full or trimmed head")
    if a.topk and not 1 <= a.topk <= L.LMH_MAX_TOPK:
        raise SystemExit(f"bench.py: --topk must be 1..{L.LMH_MAX_TOPK}")
    if a.indexed:
        if ids is None or a.full or quantized:
            raise SystemExit("bench.py: --indexed needs a shortlist config (1, 3, 4, 5), without --full, "
                             "--fp8, --mxfp4 or --nvfp4")
        workload = (f"{c.name}: M={m} K={c.k} {rows} listed rows read in place from the full head "
                    f"N={c.n} ({copies} rotated copies of W)")
    if a.fp8:
        if trimmed:
            copies = max(1, -(-2 * MALL_BYTES // (rows * c.k)) + 1)
            workload = f"{c.name}: M={m} K={c.k} trimmed to {rows} rows ({copies} rotated copies)"
        workload += ", FP8 E4M3 head (fp32 row scale)"
    if a.mxfp4:
        if kpath != "mfma":
            raise SystemExit("bench.py: MXFP4 heads run on the matrix-core path only")
        if trimmed:
            copies = max(1, -(-2 * MALL_BYTES // head_bytes(rows, c.k, "mxfp4")) + 1)
            workload = f"{c.name}: M={m} K={c.k} trimmed to {rows} rows ({copies} rotated copies)"
        workload += ", MXFP4 head (E2M1, E8M0 scale per 32)"
    if a.nvfp4:
        if kpath != "mfma":
            raise SystemExit("bench.py: NVFP4 heads run on the matrix-core path only")
        if trimmed:
            copies = max(1, -(-2 * MALL_BYTES // head_bytes(rows, c.k, "nvfp4")) + 1)
            workload = f"{c.name}: M={m} K={c.k} trimmed to {rows} rows ({copies} rotated copies)"
        workload += ", NVFP4 head (E2M1, E4M3 scale per 16, fp32 head scale)"
    fmt = "fp8" if a.fp8 else ("mxfp4" if a.mxfp4 else ("nvfp4" if a.nvfp4 else "bf16"))
    kname = kernel_name(kpath, m, a.indexed) if fmt == "bf16" else ("proj_mfma" if kpath == "mfma" else "proj_valu_fp8")
    return dict(inp=inp, c=c, m=m, ids=ids, trimmed=trimmed, path=path, kpath=kpath, rows=rows,
                copies=copies, workload=workload, kname=kname, fmt=fmt)


def measured_traffic(path: str, workload: str):
    """HBM bytes per projection launch from committed rocprofv3 counter
    runs, if they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    for e in table.get("entries", []):
        if e.get("path") == path and e.get("workload") == workload:
            if e.get("source_sha256_16") != source_digest():
                return None
            return e.get("bytes_projection_kernel")
    return None


def _counter_medians(csv_path: str, counter: str) -> dict:
    """Median counter value (KiB per dispatch) by kernel, from a rocprofv3
    --pmc ... --output-format csv counter_collection file."""
    import csv
    import statistics
    vals: dict = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"].replace("(anonymous namespace)::", "")
            name = name.split("(")[0].replace("void ", "").strip()
            vals.setdefault(name, []).append(float(row["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def _pick(med: dict, prefix: str):
    hits = [(k, v) for k, v in med.items() if k.startswith(prefix)]
    if len(hits) != 1:
        raise SystemExit(f"bench.py: expected one kernel named {prefix}*, found {[k for k, _ in hits]}")
    return hits[0]


def record_traffic(a, d, fetch_csv: str, write_csv: str) -> int:
    """Turn two counter runs of `bench.py --calibrate` (FETCH_SIZE, then
    WRITE_SIZE) into the entry of profiles/traffic.json for this workload.
    FETCH_SIZE and WRITE_SIZE are scaled by what they read for copy16 over
    1 GiB (1 GiB read, 1 GiB written) in the same process."""
    fm = _counter_medians(fetch_csv, "FETCH_SIZE")
    wm = _counter_medians(write_csv, "WRITE_SIZE")
    kname, fk = _pick(fm, d["kname"])
    _, wk = _pick(wm, d["kname"])
    _, ffin = _pick(fm, "finalize_argmax")
    _, wfin = _pick(wm, "finalize_argmax")
    _, fcopy = _pick(fm, "copy16")
    _, wcopy = _pick(wm, "copy16")
    gib = float(1 << 30)
    fs, ws = gib / (fcopy * 1024), gib / (wcopy * 1024)
    proj = fk * 1024 * fs + wk * 1024 * ws
    fin = ffin * 1024 * fs + wfin * 1024 * ws
    entry = {
        "path": d["kpath"], "kernel": kname, "workload": d["workload"],
        "source_sha256_16": source_digest(),
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
        "finalize_fetch_kib": ffin, "finalize_write_kib": wfin,
        "copy16_fetch_kib": fcopy, "copy16_write_kib": wcopy,
        "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
        "bytes_projection_kernel": int(round(proj)), "bytes_finalize_kernel": int(round(fin)),
        "algorithmic_bytes_projection_kernel": projection_bytes(d["m"], d["rows"], d["c"].k, d["fmt"], a.indexed),
    }
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table["about"] = ("HBM bytes per launch of the projection kernel from rocprofv3 --pmc FETCH_SIZE and "
                      "WRITE_SIZE runs of bench.py --calibrate, each scaled by what the counter reads for "
                      "copy16 over 1 GiB in the same process; valid only for the kernel source whose code "
                      "(comments excluded) has this digest")
    entries = [e for e in table.get("entries", [])
               if not (e.get("path") == entry["path"] and e.get("workload") == entry["workload"])]
    entries.append(entry)
    table["entries"] = entries
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")
    print(json.dumps(entry))
    return 0


def traffic_table() -> int:
    """profiles/traffic.json as a markdown table: per workload, the median
    counter values per dispatch, the scaled HBM bytes of one projection
    launch against the algorithmic bytes, and whether the entry was taken on
    the kernel source as it stands."""
    with open(TRAFFIC_FILE) as f:
        table = json.load(f)
    digest = source_digest()
    print("| Workload | Kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | Algorithmic bytes "
          "| Excess | Current source |")
    print("|---|---|---|---|---|---|---|---|")
    for e in table.get("entries", []):
        alg = e["algorithmic_bytes_projection_kernel"]
        got = e["bytes_projection_kernel"]
        print(f"| {e['workload']} | `{e['kernel']}` | {e['fetch_kib_per_dispatch']:,.1f} | "
              f"{e['write_kib_per_dispatch']:,.1f} | {got:,} | {alg:,} | {100 * (got / alg - 1):+.3f}% | "
              f"{'yes' if e['source_sha256_16'] == digest else 'no'} |")
    e0 = (table.get("entries") or [{}])[0]
    if e0:
        print(f"\nScale factors from copy16 over 1 GiB in each run: FETCH_SIZE x {e0['fetch_scale']}, "
              f"WRITE_SIZE x {e0['write_scale']}.")
    return 0


def blas_threads() -> dict:
    """The BLAS library numpy calls (name and version, from threadpoolctl)
    and the threads it runs: the cores the oracle's fp64 matrix products
    actually use."""
    import numpy  # noqa: F401  (loads the BLAS library threadpoolctl inspects)
    from threadpoolctl import threadpool_info
    libs = [d for d in threadpool_info() if d.get("user_api") == "blas"] or threadpool_info()
    if not libs:
        return {"library": "unknown", "threads": 1}
    top = max(libs, key=lambda d: d.get("num_threads", 1))
    name = f"{top.get('internal_api', top.get('prefix', 'blas'))} {top.get('version') or ''}".strip()
    return {"library": name, "threads": int(top.get("num_threads", 1))}


def cpu_baseline(h_np, w_np, d2t_np, budget_s: float, indexed: bool = False):
    """The fp64 oracle timed on host cores over whole calls until `budget_s`
    (indexed: the oracle reads the listed rows of the full head in place)."""
    import oracle
    blas = blas_threads()
    threads = blas["threads"]
    calls = 0
    t0 = time.perf_counter()
    while True:
        if indexed:
            oracle.oracle_project_argmax_indexed(h_np, w_np, d2t_np)
        else:
            oracle.oracle_project_argmax(h_np, w_np, d2t_np)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 50:
            break
    rows = d2t_np.size if indexed else w_np.shape[0]
    return {"value": calls / el, "unit": "calls/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "host_cpus_usable": len(os.sched_getaffinity(0)),
            "blas": blas["library"], "blas_threads": threads,
            "seconds_per_call": el / calls,
            "gbps": round(rows * w_np.shape[1] * 2 * calls / el / 1e9, 3),  # bf16 head bytes per second
            "sample": f"{calls} whole oracle calls (fp64, M={h_np.shape[0]}, "
                      f"{d2t_np.size if indexed else w_np.shape[0]} rows x K={w_np.shape[1]}) in {el:.1f} s; "
                      f"numpy + {blas['library']} with {threads} threads"}


def shortlist_ops(synth, L, torch, np, dev) -> dict:
    """Load-time and maintenance calls on the shortlisted-head workloads:
    the gather of each list (whole lmhead_trim call, host range check
    included), the device union of the two lists behind the 52,755-id list,
    and 600 escaped ids written into spare rows of the 32,768-id head."""
    stream = torch.cuda.current_stream(dev)
    w_np = synth.make_config(2)["W"]
    w = torch.from_numpy(np.array(w_np.view(np.int16))).to(dev)   # a writable copy of the read-only array
    k = w.shape[1]
    out = {"mode": "shortlist-ops", "K": k, "N": w.shape[0]}

    def events(fn, reps):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    for cfg in (3, 4, 5):
        ids = torch.from_numpy(synth.make_config(cfg)["ids"].astype(np.int32)).to(dev)
        dst = torch.empty((ids.shape[0], k), dtype=w.dtype, device=dev)
        L.lmhead_trim(w, ids, dst)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 5
        for _ in range(reps):
            L.lmhead_trim(w, ids, dst)
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / reps * 1e6
        out[f"trim_{ids.shape[0]}_us"] = round(us, 1)
        out[f"trim_{ids.shape[0]}_gbps"] = round(2 * ids.shape[0] * k * 2 / (us / 1e6) / 1e9, 1)
        del dst
    a, b, _ = synth.union_parts()
    ad, bd = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    uo = torch.empty(a.size + b.size, dtype=torch.int32, device=dev)
    uc = torch.empty(4, dtype=torch.int32, device=dev)
    out["union_us"] = round(events(lambda: L.lmhead_shortlist_union(ad, bd, w.shape[0], uo, uc), 50), 2)
    out["union_counts"] = [int(x) for x in uc.cpu().tolist()]
    ids32 = synth.make_config(4)["ids"]
    spare = 1024
    cap_ids = torch.from_numpy(np.concatenate([ids32, np.zeros(spare, np.int32)]).astype(np.int32)).to(dev)
    wt = L.lmhead_trim(w, cap_ids)
    rng = np.random.default_rng(70)
    esc = np.setdiff1d(rng.integers(0, w.shape[0], size=800), ids32)[:600].astype(np.int32)
    rows = torch.from_numpy((ids32.size + np.arange(esc.size)).astype(np.int32)).to(dev)
    escd = torch.from_numpy(esc).to(dev)
    us = events(lambda: L.lmhead_shortlist_overwrite(w, wt, cap_ids, rows, escd), 50)
    out["overwrite_600_us"] = round(us, 2)
    out["overwrite_600_gbps"] = round(2 * esc.size * k * 2 / (us / 1e6) / 1e9, 1)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--m", type=int, default=None, help="hidden rows (default: the config's first)")
    ap.add_argument("--full", action="store_true", help="project the full head even for a shortlist config")
    ap.add_argument("--path", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed regions of --steps calls (the first gives `value`; all give the spread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-read", action="store_true",
                    help="also time the plain streaming-read kernel over W (practical ceiling)")
    ap.add_argument("--calibrate", action="store_true",
                    help="after the timed region, run the plain copy and read kernels over 1 GiB "
                         "(known bytes, for scaling hardware counters)")
    ap.add_argument("--fp8", action="store_true",
                    help="quantize the head (or shortlist) to FP8 E4M3 with one scale per row at load "
                         "and time draft_project_argmax_fp8 (no CPU baseline)")
    ap.add_argument("--mxfp4", action="store_true",
                    help="quantize the head (or shortlist) to MXFP4 at load and time "
                         "draft_project_argmax_mxfp4 (no CPU baseline)")
    ap.add_argument("--nvfp4", action="store_true",
                    help="quantize the head (or shortlist) to NVFP4 at load and time "
                         "draft_project_argmax_nvfp4 (no CPU baseline)")
    ap.add_argument("--indexed", action="store_true",
                    help="read the shortlist's rows in place from the full head "
                         "(draft_project_argmax_indexed), rotating copies of W past the Infinity Cache")
    ap.add_argument("--topk", type=int, default=0,
                    help="time the top-k call (draft_project_topk, or its FP8 / MXFP4 form) with this k "
                         "instead of the argmax; whole calls only")
    ap.add_argument("--logits", choices=["rows", "vocab"], default=None,
                    help="time draft_project_logits instead of the argmax: every logit as [M, R] (rows), "
                         "or scattered through d2t into [M, N] with -inf elsewhere (vocab; the full head "
                         "takes d2t = 0..N-1); bf16 heads; whole calls only")
    ap.add_argument("--sweep-m", default="",
                    help="comma-separated hidden-row counts: time the projection kernel of the argmax on "
                         "both kernels (VALU where it takes the shape, matrix cores) at each, on this "
                         "workload's head, one JSON line per (M, kernel); for locating the crossover under "
                         "rocprofv3")
    ap.add_argument("--rows", type=int, default=0,
                    help="time draft_project_argmax_keys over the first ROWS rows of the full head (one GPU's "
                         "share of a vocabulary split: 124160 at 2 GPUs, 31040 at 8), rotating copies past "
                         "the Infinity Cache")
    ap.add_argument("--fused", action="store_true",
                    help="time the argmax as one launch per call (draft_project_argmax_fused: workgroups merge "
                         "their keys with atomics, the last one writes the outputs) instead of the projection + "
                         "fold pair; bf16 heads; whole calls only")
    ap.add_argument("--unprepared", action="store_true",
                    help="call the argmax through the plain binding (every tensor checked on every call) "
                         "instead of the prepared calls (PreparedArgmax and its FP8 / MXFP4 / NVFP4 forms)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the --steps calls of a timed region in one HIP graph and time its replays "
                         "(the calls without the host's launch cost)")
    ap.add_argument("--shortlist-ops", action="store_true",
                    help="instead of the projection: time the list gathers, the device union of two lists "
                         "and 600 escaped ids written into spare rows (one JSON line)")
    ap.add_argument("--traffic-table", action="store_true",
                    help="no GPU: print profiles/traffic.json as a markdown table (one row per workload)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: write this workload's entry of profiles/traffic.json from the "
                         "counter_collection.csv files of two rocprofv3 --pmc runs (FETCH_SIZE, "
                         "WRITE_SIZE) of bench.py --calibrate with the same workload options")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {a.gpus} is not supported "
              "(the projection shards by vocabulary rows with one small all-reduce, "
              "which is not built here)", file=sys.stderr)
        return 2

    if a.traffic_table:
        return traffic_table()

    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import synth
    from vocab_shortlisted_lm_amd import lmhead as L

    L.lib()
    d = describe(a, synth, L)
    if a.record_traffic:
        return record_traffic(a, d, *a.record_traffic)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.shortlist_ops:
        print(json.dumps(shortlist_ops(synth, L, torch, np, dev)), flush=True)
        return 0

    inp, c, m, ids, trimmed, path = d["inp"], d["c"], d["m"], d["ids"], d["trimmed"], d["path"]
    rows, workload, kpath = d["rows"], d["workload"], d["kpath"]
    h_np = inp["h"][m] if m in inp["h"] else synth.hidden(c.h_seed[0], 0, m, c.k)
    w_np = inp["W"]

    # writable copies: the seeded arrays are read-only and torch.from_numpy wants a writable buffer
    w_full = torch.from_numpy(np.array(w_np.view(np.int16))).to(dev)
    h = torch.from_numpy(np.array(h_np.view(np.int16))).to(dev)
    if a.rows:
        d2t = None
        heads = [w_full[:rows].clone() for _ in range(d["copies"])] if d["copies"] > 1 else [w_full[:rows]]
        if d["copies"] > 1:
            del w_full
        out_key = torch.empty(m, dtype=torch.int64, device=dev)
    elif a.indexed:
        d2t = torch.from_numpy(ids.astype(np.int32)).to(dev)
        heads = [w_full] + [w_full.clone() for _ in range(d["copies"] - 1)]
    elif trimmed:
        d2t = torch.from_numpy(ids.astype(np.int32)).to(dev)
        heads = [L.lmhead_trim(w_full, d2t) for _ in range(d["copies"])]
        del w_full
    else:
        d2t = None
        heads = [w_full]
    if a.fp8:
        qheads = []
        for w in heads:
            qheads.append(L.lmhead_quantize_fp8(w))
            torch.cuda.synchronize()
        del heads, w
        heads = qheads
    if a.mxfp4:
        qheads = []
        for w in heads:
            qheads.append(L.lmhead_quantize_mxfp4(w))
            torch.cuda.synchronize()
        del heads, w
        heads = qheads
    if a.nvfp4:
        qheads = []
        for w in heads:
            qheads.append(L.lmhead_quantize_nvfp4(w))
            torch.cuda.synchronize()
        del heads, w
        heads = qheads
    torch.cuda.synchronize()

    ws = L.new_workspace(dev)
    if a.sweep_m:
        if d["fmt"] != "bf16" or a.indexed or a.topk or a.logits or a.fused or a.rows:
            raise SystemExit("bench.py: --sweep-m times the bf16 argmax over a full or trimmed head")
        stream = torch.cuda.current_stream(dev)
        for ms in [int(x) for x in a.sweep_m.split(",")]:
            hm = torch.from_numpy(np.array(synth.hidden(c.h_seed[0] + 97, 0, ms, c.k).view(np.int16))).to(dev)
            oid = torch.empty(ms, dtype=torch.int32, device=dev)
            olg = torch.empty(ms, dtype=torch.float32, device=dev)
            for pname, pv in (("valu", L.LMH_PATH_VALU), ("mfma", L.LMH_PATH_MFMA)):
                if pv == L.LMH_PATH_VALU and not (ms <= 8 and ms * ((c.k // 8 + 63) // 64) <= 40):
                    continue
                L.lmhead_bench_time_argmax(hm, heads, d2t, pv, max(1, a.warmup), oid, olg, ws, stream)
                t = [L.lmhead_bench_time_argmax(hm, heads, d2t, pv, a.steps, oid, olg, ws, stream)
                     for _ in range(max(1, a.repeats))]
                print(json.dumps({"mode": "kernel sweep", "workload": workload, "M": ms, "path": pname,
                                  "kernel": kernel_name(pname, ms), "rows": rows,
                                  "auto_path": {L.LMH_PATH_VALU: "valu", L.LMH_PATH_MFMA: "mfma"}[
                                      L.draft_project_auto_path_rows(ms, c.k, rows)],
                                  "kernel_avg_us": round(float(np.median(t)) * 1e3, 2),
                                  "spread_us": [round(min(t) * 1e3, 2), round(max(t) * 1e3, 2)],
                                  "launches": a.steps, "regions": len(t)}), flush=True)
        return 0
    out_id = torch.empty(m, dtype=torch.int32, device=dev)
    out_logit = torch.empty(m, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    launch_on = [stream]   # the stream the calls go to (a capture stream under --graph)
    out_bytes = 8 * m
    if a.topk:
        tk_id = torch.empty((m, a.topk), dtype=torch.int32, device=dev)
        tk_logit = torch.empty((m, a.topk), dtype=torch.float32, device=dev)
        tk_ws = torch.empty(L.draft_project_topk_workspace_bytes(m, a.topk), dtype=torch.uint8, device=dev)
        out_bytes = 8 * m * a.topk
    if a.logits:
        lg_d2t = None
        if a.logits == "vocab":
            lg_d2t = d2t if d2t is not None else torch.arange(c.n, dtype=torch.int32, device=dev)
        lg_cols = c.n if lg_d2t is not None else rows
        lg_out = torch.empty((m, lg_cols), dtype=torch.float32, device=dev)
        out_bytes = 4 * m * lg_cols

    if a.fused:
        state = L.new_state(dev)

    # The argmax (bf16, its single-launch form, and over quantized heads)
    # goes through the prepared calls, as a decode loop would make them: the
    # buffers are checked once, then each step is one C call.  One prepared
    # step per rotated head copy and per stream (the capture stream under
    # --graph is another).
    prepared: dict = {}

    def make_prepared(w, st):
        if a.fp8:
            return L.PreparedArgmaxFp8(h, w[0], w[1], d2t, path, out_id, out_logit, ws, st)
        if a.mxfp4:
            return L.PreparedArgmaxMxfp4(h, w[0], w[1], d2t, path, out_id, out_logit, ws, st)
        if a.nvfp4:
            return L.PreparedArgmaxNvfp4(h, w[0], w[1], w[2], d2t, path, out_id, out_logit, ws, st)
        return L.PreparedArgmax(h, w, d2t, path, out_id, out_logit, ws, st, state=state if a.fused else None)

    def prepared_step(i):
        st = launch_on[0]
        steps_ = prepared.get(id(st))
        if steps_ is None:
            steps_ = [make_prepared(w, st) for w in heads]
            prepared[id(st)] = steps_
        steps_[i % len(steps_)]()

    def step(i):
        if a.rows:
            L.draft_project_argmax_keys(h, heads[i % len(heads)], 0, path, out_key, ws, launch_on[0])
        elif a.fused and not a.unprepared:
            prepared_step(i)
        elif a.fused:
            L.draft_project_argmax_fused_path(h, heads[i % len(heads)], d2t, path, state, out_id, out_logit,
                                              launch_on[0])
        elif a.topk:
            if a.fp8:
                q, sc = heads[i % len(heads)]
                L.draft_project_topk_fp8(h, q, sc, d2t, a.topk, tk_id, tk_logit, tk_ws, path, launch_on[0])
            elif a.mxfp4:
                q, sc = heads[i % len(heads)]
                L.draft_project_topk_mxfp4(h, q, sc, d2t, a.topk, tk_id, tk_logit, tk_ws, path, launch_on[0])
            elif a.nvfp4:
                q, sc, gs = heads[i % len(heads)]
                L.draft_project_topk_nvfp4(h, q, sc, gs, d2t, a.topk, tk_id, tk_logit, tk_ws, path, launch_on[0])
            else:
                L.draft_project_topk(h, heads[i % len(heads)], d2t, a.topk, tk_id, tk_logit, tk_ws, path, launch_on[0])
        elif a.logits:
            L.draft_project_logits(h, heads[i % len(heads)], lg_d2t, c.n if lg_d2t is not None else None,
                                   lg_out, path, launch_on[0])
        elif a.indexed:
            L.draft_project_argmax_indexed(h, heads[i % len(heads)], d2t, path, out_id, out_logit, ws, launch_on[0])
        elif (a.fp8 or a.mxfp4 or a.nvfp4) and not a.unprepared:
            prepared_step(i)
        elif a.fp8:
            q, sc = heads[i % len(heads)]
            L.draft_project_argmax_fp8(h, q, sc, d2t, path, out_id, out_logit, ws, launch_on[0])
        elif a.mxfp4:
            q, sc = heads[i % len(heads)]
            L.draft_project_argmax_mxfp4(h, q, sc, d2t, path, out_id, out_logit, ws, launch_on[0])
        elif a.nvfp4:
            q, sc, gs = heads[i % len(heads)]
            L.draft_project_argmax_nvfp4(h, q, sc, gs, d2t, path, out_id, out_logit, ws, launch_on[0])
        elif not a.unprepared:
            prepared_step(i)
        else:
            L.draft_project_argmax_path(h, heads[i % len(heads)], d2t, path, out_id, out_logit, ws,
                                        launch_on[0])

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if a.graph:
        # the timed region's calls, captured once; a region is then one replay
        cap = torch.cuda.Stream(dev)
        graph = torch.cuda.CUDAGraph()
        launch_on[0] = cap
        with torch.cuda.graph(graph, stream=cap):
            for i in range(a.steps):
                step(i)
        launch_on[0] = stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()

    def region():
        if graph is not None:
            graph.replay()
        else:
            for i in range(a.steps):
                step(i)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    region()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / a.steps
    calls_per_s = a.steps / (ms_total / 1e3)

    # The same timed region again, for the spread of the rate (the first
    # region alone gives `value`).
    rates = [calls_per_s]
    for _ in range(max(0, a.repeats - 1)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        region()
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(a.steps / (e0.elapsed_time(e1) / 1e3))

    if a.topk or a.logits or a.fused:
        # whole calls only: the kernel-only timer covers the argmax epilogue
        result = {
            "mode": f"top-{a.topk}" if a.topk else (f"logits ({a.logits})" if a.logits else "argmax, single launch (fused)"),
            "workload": workload, "M": m, "K": c.k, "rows": rows, "fmt": d["fmt"], "graph": a.graph,
            "steps": a.steps,
            "warmup": a.warmup, "us_per_call": round(ms_per_step * 1e3, 2),
            "repeats_us_per_call": {"median": round(float(np.median([1e6 / r for r in rates])), 2),
                                    "p10": round(float(np.percentile([1e6 / r for r in rates], 10)), 2),
                                    "p90": round(float(np.percentile([1e6 / r for r in rates], 90)), 2),
                                    "n": len(rates)},
            "bytes_per_call": projection_bytes(m, rows, c.k, d["fmt"]) + out_bytes,
        }
        result["gbps"] = round(result["bytes_per_call"] / (ms_per_step / 1e3) / 1e9, 1)
        print(json.dumps(result), flush=True)
        return 0

    # The projection kernel alone: as many launches again, back to back on
    # this stream between two HIP events the library records (no fold).
    if a.indexed:
        proj_ms = L.lmhead_bench_time_argmax_indexed(h, heads, d2t, path, a.steps, out_id, out_logit, ws, stream)
    elif a.fp8:
        proj_ms = L.lmhead_bench_time_argmax_fp8(h, heads, d2t, path, a.steps, out_id, out_logit, ws, stream)
    elif a.mxfp4:
        proj_ms = L.lmhead_bench_time_argmax_mxfp4(h, heads, d2t, path, a.steps, out_id, out_logit, ws, stream)
    elif a.nvfp4:
        proj_ms = L.lmhead_bench_time_argmax_nvfp4(h, heads, d2t, path, a.steps, out_id, out_logit, ws, stream)
    else:
        proj_ms = L.lmhead_bench_time_argmax(h, heads, d2t, path, a.steps, out_id, out_logit, ws, stream)
    # a rotated workload also timed on one copy, which the Infinity Cache can hold
    proj_ms_hot = None
    if len(heads) > 1:
        one = heads[:1]
        if a.indexed:
            proj_ms_hot = L.lmhead_bench_time_argmax_indexed(h, one, d2t, path, a.steps, out_id, out_logit, ws, stream)
        elif a.fp8:
            proj_ms_hot = L.lmhead_bench_time_argmax_fp8(h, one, d2t, path, a.steps, out_id, out_logit, ws, stream)
        elif a.mxfp4:
            proj_ms_hot = L.lmhead_bench_time_argmax_mxfp4(h, one, d2t, path, a.steps, out_id, out_logit, ws, stream)
        elif a.nvfp4:
            proj_ms_hot = L.lmhead_bench_time_argmax_nvfp4(h, one, d2t, path, a.steps, out_id, out_logit, ws, stream)
        else:
            proj_ms_hot = L.lmhead_bench_time_argmax(h, one, d2t, path, a.steps, out_id, out_logit, ws, stream)
    pbytes = projection_bytes(m, rows, c.k, d["fmt"], a.indexed)
    achieved = pbytes / (proj_ms / 1e3) / 1e9
    abytes = algorithmic_bytes(m, rows, c.k, d2t is not None, d["fmt"], a.indexed)
    traffic = measured_traffic(kpath, workload)
    extra = {}
    if a.stream_read:
        # the plain streaming read over the same head bytes (codes only for a
        # quantized head), rotating through the same copies as the calls
        sink = torch.zeros(L.lmhead_bench_sink_words(), dtype=torch.int32, device=dev)
        bufs = [hd[0] if d["fmt"] != "bf16" else hd for hd in heads]
        n_sr = 20 * len(bufs)
        for i in range(3):
            L.lmhead_bench_stream_read(bufs[i % len(bufs)], sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_sr):
            L.lmhead_bench_stream_read(bufs[i % len(bufs)], sink)
        e1.record(stream)
        torch.cuda.synchronize()
        nb = bufs[0].numel() * bufs[0].element_size()
        sr_us = e0.elapsed_time(e1) / n_sr * 1e3
        extra["stream_read"] = {"bytes": nb, "us": round(sr_us, 2), "gbps": round(nb / (sr_us / 1e6) / 1e9, 1),
                                "copies": len(bufs)}

    if a.calibrate:
        nb = 1 << 30
        src = torch.empty(nb // 4, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty_like(src)
        sink = torch.zeros(L.lmhead_bench_sink_words(), dtype=torch.int32, device=dev)
        for _ in range(3):
            L.lmhead_bench_copy(src, dst)
        for _ in range(3):
            L.lmhead_bench_stream_read(src, sink)
        torch.cuda.synchronize()
        extra["calibration"] = {"copy_bytes_read": nb, "copy_bytes_written": nb, "read_bytes": nb,
                                "dispatches": "3 x copy16, then 3 x stream_read"}
        del src, dst

    result = {
        "metric": METRIC,
        "value": round(calls_per_s, 2),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "e4m3 W x bf16 h, fp32 accumulate", "mxfp4": "mxfp4 (e2m1 + e8m0) W x bf16 h, fp32 accumulate",
                  "nvfp4": "nvfp4 (e2m1 + e4m3 per 16 + fp32) W x bf16 h, fp32 accumulate",
                  "bf16": "bf16"}[d["fmt"]],
        "data": "synthetic (seeded bf16 W ~ N(0, 0.02), h ~ N(0, 1))",
        "config": {"workload": workload, "M": m, "K": c.k, "rows": rows, "indexed": a.indexed,
                   "kernel": d["kname"], "d2t": d2t is not None, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "kernel": d["kname"],
                     "kernel_avg_us": round(proj_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": pbytes,
                     "step_gbps": round(abytes / (ms_per_step / 1e3) / 1e9, 1),
                     "algorithmic_bytes_per_step": abytes},
        "wall_s": round(wall, 3),
        "graph": a.graph,
        "repeats": {"n": len(rates), "unit": "calls/s", "median": round(float(np.median(rates)), 2),
                    "p10": round(float(np.percentile(rates, 10)), 2),
                    "p90": round(float(np.percentile(rates, 90)), 2)},
    }
    if proj_ms_hot is not None:
        result["mall"] = {"copies": len(heads), "kernel_avg_us_rotated": round(proj_ms * 1e3, 2),
                          "kernel_avg_us_one_copy": round(proj_ms_hot * 1e3, 2)}
    result.update(extra)
    if not a.no_cpu_baseline and d["fmt"] == "bf16":
        hb = h_np
        if a.indexed:
            result["cpu_baseline"] = cpu_baseline(hb, w_np, ids, a.cpu_seconds, indexed=True)
        else:
            wb = w_np[ids] if trimmed else (w_np[:rows] if a.rows else w_np)
            result["cpu_baseline"] = cpu_baseline(hb, wb, ids if trimmed else None, a.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
