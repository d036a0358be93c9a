#!/usr/bin/env python3
"""Throughput of the packed-sequence (THD) metadata path on one MI355X.

One step is one ``psq_process_thd`` call on the pipeline-stage embedding
workload: a document map int32 [32, 32768] (docs of length U{1..24},
trailing pad U{0..16} per row) with bf16 hidden states [32, 32768, 4096]
and int64 position ids, collapsed to THD [1048576, 4096] with cu_seqlens,
max_seqlen and the padding mask -- the map kernel, then the collapse copy.
Inputs are resident in HBM before timing starts.  The other four workloads
are timed too and reported under ``per_config`` (the document maps [4, 64]
and [8, 4096], the length tables with 3 collapsed int64 tensors, and the
squeeze of 65536 sources into 16384-slot packs), and so are the steps around
them: the length tables split into 4 row groups, the metadata-free padding
mask of a 131072-id stream, and the trainer's squeeze of a 256-row padded
rectangle into token-budget bins.  Every workload's outputs are compared bit
for bit with the CPU oracle after timing.

Prints one JSON line.  ``roofline`` relates the algorithmic bytes of one
call (each input read once, each output written once) to the call's
average duration from HIP events on the launch stream; ``cpu_baseline`` is
the CPU oracle on a bounded sample of the same workload, on one host core.
Each per-config line gives the time of an isolated call (HIP events around
it; for the latency-bound workloads this includes the launch) and, for the
workloads timed without a cache flush, ``us_back_to_back``: the time per
call of a stream of calls enqueued without waiting, so that each launch
overlaps the previous call, and ``us_in_graph``: the time per call of 20
calls captured in one HIP graph and replayed.  ``launch_floor`` times the
library's smallest launch the same three ways: the floor under the
latency-bound workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
METRIC = "packed tokens/sec (G tok/s) + achieved HBM GB/s vs MI355X peak, per config"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_stage_embedding.json")


# the sources of the stage-embedding step's two kernels (the one-launch map
# k_doc_small, then the collapse copy k_copies)
STAGE_KERNEL_SOURCES = ("k_segments.hip", "k_copy.hip", "psq_copy.hpp", "psq_device.hpp")

# launch grids (work-items) of the stage step's kernels: 256 map tiles of 256
# threads, and one 64-lane workgroup per KiB of the 8 GiB + 8 MiB collapse
STAGE_GRIDS = {"psq::k_doc_small<int, 4>": "65536",
               "psq::k_copies<u32x4, true>": "537395200"}
# the 1 GiB calibration copy: a one-token map, then 2^26 copy lanes
CALIB_GRID = str((1 << 30) // 16)

# per-config workloads whose launch has a grid no other launch of a counter run
# shares, and the sources that kernel is built from (the doc_map_small map
# shares its grid with the calibration copy's one-token map, and thd_split_4
# its grid with thd_tables, so neither is listed)
WORKLOAD_COUNTERS = {
    "pack_sources": ("psq::k_pack_rows<896u> [grid 4263296]", ("k_pack.hip", "psq_device.hpp")),
    "trainer_rectangle": ("psq::k_pack_rows<256u> [grid 61440]", ("k_pack.hip", "psq_device.hpp")),
    "pad_tail_stream": ("psq::k_pad_ids<long> [grid 16384]", ("k_padids.hip", "psq_device.hpp")),
    "doc_map_medium": ("psq::k_doc_small<int, 1> [grid 8192]", ("k_segments.hip", "psq_device.hpp")),
}


# rows of profiles/hbm_traffic_counters.md: (label, counter key, workload whose
# algorithmic bytes the row is measured against; the stage step's two launches
# are split into the collapse copy and the map)
COUNTER_TABLE = [
    ("k_copies<u32x4, true> (stage_embedding, launch 2: the collapse)",
     "psq::k_copies<u32x4, true> [grid 537395200]", "stage_copy"),
    ("k_doc_small<int, 4> (stage_embedding, launch 1: the map)",
     "psq::k_doc_small<int, 4> [grid 65536]", "stage_map"),
    ("stage_embedding step (both launches)", None, "stage_embedding"),
    ("k_pack_rows<896> (pack_sources)", WORKLOAD_COUNTERS["pack_sources"][0], "pack_sources"),
    ("k_pack_rows<256> (trainer_rectangle)", WORKLOAD_COUNTERS["trainer_rectangle"][0],
     "trainer_rectangle"),
    ("k_thd_small<long, 0> (thd_tables and thd_split_4: same grid, medians merged)",
     "psq::k_thd_small<long, 0> [grid 214016]", "thd_tables"),
    ("k_pad_ids<long> (pad_tail_stream)", WORKLOAD_COUNTERS["pad_tail_stream"][0],
     "pad_tail_stream"),
    ("k_doc_small<int, 1> (doc_map_medium)", WORKLOAD_COUNTERS["doc_map_medium"][0],
     "doc_map_medium"),
]

COUNTERS_MD = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
COUNTER_COMMANDS = """rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc_fetch -o fetch -- python3 bench.py --profile-launches 3 --launch-info rocprof_out/launch_info.json
rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc_write -o write -- python3 bench.py --profile-launches 3
python bench.py --summarize-counters rocprof_out/pmc_fetch/fetch_counter_collection.csv rocprof_out/pmc_write/write_counter_collection.csv --launch-info rocprof_out/launch_info.json"""

COUNTERS_NOTES = """Per-kernel values are medians over the launches. `profiles/traffic_stage_embedding.json`
holds the full output, tagged with the hash of the stage kernels' code. bench.py uses
it for the headline `roofline.traffic` only while that code is unchanged.

Its `workloads` entries carry the same figure for per-config lines whose launch grid no
other launch of the run shares: pack_sources, trainer_rectangle, pad_tail_stream and
doc_map_medium. Each is tagged with a hash of its own kernel's code, and bench.py
reports it as that line's `roofline.traffic` under the same rule. doc_map_small's map
shares its grid with the calibration copy's one-token map, and thd_split_4 shares its
grid with thd_tables, so their traffic stays null.

The calibration factor holds for launches that spread over every memory channel. Below
about 1 MB, the scaled FETCH_SIZE is dominated by fixed per-launch reads: kernel code,
arguments, the workspace header and the look-back descriptors. doc_map_medium's ratio is
that overhead on a 128 KiB map, not re-reads. For the two large kernels the counters
match the algorithmic bytes to within 2 %.

The squeeze moves about 1.5 % more than its algorithmic bytes, all of it on the read
side. Pad slots re-read a token of their own member, which keeps the loads straight-line
code. Most of those re-reads hit lines already in flight; the rest is the excess."""


def write_counters_md(out: dict, algo: dict) -> None:
    """profiles/hbm_traffic_counters.md from the scaled counters and the
    algorithmic bytes that the counter run's own workloads reported."""
    fmt = lambda x: f"{x:,.0f}".replace(",", " ")
    ks = out["kernels"]
    cal = ks["calibration_copy_1GiB"]
    cross = out["library_copy_1GiB_cross_check"]
    lines = ["# HBM traffic from counters (FETCH_SIZE, WRITE_SIZE)", "",
             "Commands (on an MI355X, from the repository root), one counter per run:", "",
             "```", COUNTER_COMMANDS, "```", "",
             "`--profile-launches 3` first launches torch's `zero_` and `sum` over a 1 GiB "
             "int64 tensor", "(the calibration) and the library's own 1 GiB copy (the "
             "collapse path with a one-token", "map, a cross-check), three times each. It then "
             "launches each workload three times.", "The stage-embedding step is two launches: "
             "the map kernel, then the collapse copy.", "`--launch-info` records each "
             "workload's algorithmic bytes, computed by the same code as", "the bench's "
             "rooflines.", "",
             "Calibration, on kernels this library did not write, over one 1 GiB int64 tensor:",
             "",
             f"- torch `sum` reads it once: FETCH_SIZE = "
             f"{fmt(ks['calibration_sum_1GiB']['fetch_kib'])} KiB per dispatch, so read bytes = "
             f"FETCH_SIZE × 1024 × {out['fetch_scale']};",
             f"- torch `zero_` writes it once: WRITE_SIZE = "
             f"{fmt(ks['calibration_fill_1GiB']['write_kib'])} KiB per dispatch, so write bytes "
             f"= WRITE_SIZE × 1024 × {out['write_scale']}.", "",
             f"Cross-check: the library's own 1 GiB copy (FETCH_SIZE = {fmt(cal['fetch_kib'])} KiB, "
             f"WRITE_SIZE = {fmt(cal['write_kib'])} KiB) then reads {cross['read_ratio']} GiB and "
             f"writes {cross['write_ratio']} GiB per GiB copied.", "",
             "| kernel (workload) | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch | "
             "algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|"]
    for label, key, workload in COUNTER_TABLE:
        a = algo.get(workload)
        if key is None:
            b = out["bytes_per_launch"]
            lines.append(f"| {label} | | | | {fmt(b)} | {fmt(a)} | {b / a:.3f} |")
            continue
        v = out["kernels"].get(key)
        if v is None or a is None:
            continue
        grid = int(key.split("[grid ")[1].rstrip("]"))
        b = v["bytes_per_launch"]
        lines.append(f"| {label} | {fmt(grid)} | {fmt(v['fetch_kib'])} | {fmt(v['write_kib'])} | "
                     f"{fmt(b)} | {fmt(a)} | {b / a:.3f} |")
    lines += ["", COUNTERS_NOTES]
    with open(COUNTERS_MD, "w") as f:
        f.write("\n".join(lines) + "\n")


def code_text(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines: an
    edit of a comment leaves the kernel, and so its counter figures, as they
    were.  (The sources hold no string literal containing a comment opener.)"""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(names=STAGE_KERNEL_SOURCES) -> str:
    """Hash of the kernel's code: stored HBM counter figures are only used
    while the kernel they were taken on is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "varlen_attention_metadata_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name)) as f:
            h.update(name.encode() + b"\0" + code_text(f.read()).encode())
    return h.hexdigest()[:16]


def kernel_short_name(name: str) -> str:
    """psq kernel name without namespaces' noise and without its parameter list
    (vector element types are spelled u32x4)."""
    import re
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    name = re.sub(r"unsigned int __attribute__\(\(ext_vector_type\((\d+)\)\)\)", r"u32x\1", name)
    name = name.replace("unsigned int __vector(4)", "u32x4")
    return name.split("(")[0]


def summarize_counters(fetch_csv: str, write_csv: str, launch_info: str | None = None) -> None:
    """Turn two rocprofv3 --pmc runs of ``--profile-launches`` (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch) into per-kernel HBM bytes, scaled by
    what the same counters read for the 1 GiB calibration copy.  With the
    ``--launch-info`` file of the counter run, also writes the markdown table
    against each workload's algorithmic bytes."""
    import csv
    import statistics


    def load(path):
        per = {}
        torch_calib = {}       # key -> (grid, [values]) of the largest grid seen
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "psq::" not in name:
                # torch's kernels over the 1 GiB int64 tensor: the largest
                # fill of int64 and the largest sum reduction of the run
                key = ("calibration_fill_1GiB" if "FillFunctor<long>" in name else
                       "calibration_sum_1GiB" if "reduce_kernel" in name and "sum_functor" in name
                       else None)
                if key is not None:
                    g = int(r["Grid_Size"])
                    cur = torch_calib.get(key)
                    if cur is None or g > cur[0]:
                        torch_calib[key] = (g, [float(r["Counter_Value"])])
                    elif g == cur[0]:
                        cur[1].append(float(r["Counter_Value"]))
                continue
            short = kernel_short_name(name)
            # one kernel can serve several workloads: the grid tells them apart
            key = ("calibration_copy_1GiB" if r["Grid_Size"] == CALIB_GRID and "k_copies" in short
                   else f"{short} [grid {r['Grid_Size']}]")
            per.setdefault(key, []).append(float(r["Counter_Value"]))
        for key, (_, v) in torch_calib.items():
            per[key] = v
        return {k: statistics.median(v) for k, v in per.items()}

    fetch, write = load(fetch_csv), load(write_csv)
    # independent scales: reads from torch's sum, writes from torch's zero_
    f_scale = (1 << 30) / 1024 / fetch["calibration_sum_1GiB"]
    w_scale = (1 << 30) / 1024 / write["calibration_fill_1GiB"]
    rows = {}
    for k in fetch:
        if k in write:
            rb, wb = fetch[k] * f_scale * 1024, write[k] * w_scale * 1024
            rows[k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                       "read_bytes": round(rb), "write_bytes": round(wb),
                       "bytes_per_launch": round(rb + wb)}
    stage = [rows[f"{k} [grid {g}]"]["bytes_per_launch"] for k, g in STAGE_GRIDS.items()]
    workloads = {name: {"kernel": key, "source_hash": source_hash(srcs),
                        "bytes_per_launch": rows[key]["bytes_per_launch"]}
                 for name, (key, srcs) in WORKLOAD_COUNTERS.items() if key in rows}
    cal = rows.get("calibration_copy_1GiB")
    cross = None if cal is None else {
        "read_ratio": round(cal["read_bytes"] / (1 << 30), 4),
        "write_ratio": round(cal["write_bytes"] / (1 << 30), 4)}
    out = {"source_hash": source_hash(), "kernel": " + ".join(STAGE_GRIDS),
           "workload": "stage_embedding", "bytes_per_launch": sum(stage),
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "calibration": "reads: torch sum over a 1 GiB int64 tensor (FETCH_SIZE); writes: "
                          "torch zero_ of it (WRITE_SIZE)",
           "library_copy_1GiB_cross_check": cross,
           "workloads": workloads, "kernels": rows}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    if launch_info:
        with open(launch_info) as f:
            write_counters_md(out, json.load(f))
    print(json.dumps(out, indent=1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=80)     # >= 200 ms of timed work
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the bit-exact comparison of outputs with the CPU oracle")
    ap.add_argument("--per-config-iters", type=int, default=50)
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 kernel_stats.csv")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_stage_embedding.json from two rocprofv3 "
                         "--pmc runs (FETCH_SIZE, WRITE_SIZE) of --profile-launches")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="for counter runs under rocprofv3: launch every workload and a "
                         "plain 1 GiB calibration copy this many times, print no JSON")
    ap.add_argument("--launch-info", default=None,
                    help="with --profile-launches: write each workload's algorithmic bytes "
                         "to this JSON file; with --summarize-counters: read it and write "
                         "profiles/hbm_traffic_counters.md")
    return ap.parse_args()


class Timer:
    """HIP events around each launch on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        t = self.torch
        self.a = t.cuda.Event(enable_timing=True)
        self.b = t.cuda.Event(enable_timing=True)
        self.a.record(t.cuda.current_stream())
        return self

    def __exit__(self, *exc):
        self.b.record(self.torch.cuda.current_stream())
        self.pairs.append((self.a, self.b))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        v = [a.elapsed_time(b) for a, b in self.pairs]
        return sum(v) / len(v), min(v)

    def median_ms(self):
        self.torch.cuda.synchronize()
        v = sorted(a.elapsed_time(b) for a, b in self.pairs)
        return v[len(v) // 2]


# ---------------------------------------------------------------------------
# workloads: each returns (call, tokens_per_call, algorithmic_bytes, info)
# ---------------------------------------------------------------------------

def setup_stage_embedding(torch, psq, lib, synth, dev):
    B, S, H = 32, 32768, 4096
    w = synth.stage_embedding(5, B, S)
    T = B * S
    doc = torch.from_numpy(w["doc_ids"]).to(dev)
    pos = torch.from_numpy(w["position_ids"]).to(dev)
    hidden = synth.stage_hidden(5, B, S, H, dev)
    out_h = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    out_p = torch.empty(T, dtype=torch.int64, device=dev)
    cu = torch.empty(T + 1, dtype=torch.int32, device=dev)
    cp = torch.empty(T + 1, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    scal = torch.zeros(4, dtype=torch.int32, device=dev)
    layout = lib.make_layout(lib.LAYOUT_DOC_IDS, doc_ids=doc.data_ptr(), doc_dtype=lib.I32)
    copies, n_c = lib.make_copies([
        (hidden.data_ptr(), out_h.data_ptr(), 1, hidden.numel() * 2, hidden.numel() * 2),
        (pos.data_ptr(), out_p.data_ptr(), 1, pos.numel() * 8, pos.numel() * 8)])
    ws = psq.workspace_for(dev, lib.psq_process_thd_workspace(layout, B, S))
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = scal.data_ptr()

    def call(stream=stream):
        lib.psq_process_thd(layout, B, S, cu.data_ptr(), cp.data_ptr(), sp, sp + 4, sp + 8,
                            mask.data_ptr(), copies, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                            stream)

    call()
    n, mx, _, st = scal.cpu().tolist()
    assert st == 0, st
    algo = 4 * T + 4 * T * H + 16 * T + T + 8 * (n + 1) + 16
    info = {"workload": "stage_embedding", "B": B, "S": S, "H": H, "num_segments": n,
            "max_seqlen": mx}
    keep = {"doc": doc, "pos": pos, "hidden": hidden, "out": (out_h, out_p, cu, cp, mask, scal, ws),
            "host": w}
    return call, T, algo, info, keep


def setup_doc_map(torch, psq, lib, synth, dev, which):
    d = synth.doc_map_small() if which == 1 else synth.doc_map_medium()
    B, S = d.shape
    doc = torch.from_numpy(d).to(dev)
    cu = torch.empty(B * S + 1, dtype=torch.int32, device=dev)
    scal = torch.zeros(4, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, lib.psq_params_from_doc_ids_workspace(B, S))
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = scal.data_ptr()

    def call(stream=stream):
        lib.psq_params_from_doc_ids(doc.data_ptr(), lib.I32, B, S, cu.data_ptr(), sp, sp + 4,
                                    None, sp + 8, ws.data_ptr(), ws.numel(), stream)

    call()
    n = int(scal[0].item())
    algo = 4 * B * S + 4 * (n + 1) + 12
    name = "doc_map_small" if which == 1 else "doc_map_medium"
    return call, B * S, algo, {"workload": name, "B": B, "S": S, "num_segments": n}, (doc, cu, scal, ws)


def setup_thd(torch, psq, lib, synth, dev):
    w = synth.thd_tables()
    S = w["S"]
    B, P = w["seq_lens"].shape
    T = B * S
    t = {k: torch.from_numpy(w[k]).to(dev) for k in
         ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    outs = {k: torch.empty(T, dtype=torch.int64, device=dev) for k in ("input_ids", "labels", "position_ids")}
    cu = torch.empty(B * P + 1, dtype=torch.int32, device=dev)
    cp = torch.empty(B * P + 1, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    scal = torch.zeros(4, dtype=torch.int32, device=dev)
    layout = lib.make_layout(lib.LAYOUT_SEQ_LENS, t["seq_lens"].data_ptr(),
                             t["seq_lens_padded"].data_ptr(), lib.I64, P, -1000)
    copies, n_c = lib.make_copies([(t[k].data_ptr(), outs[k].data_ptr(), 1, T * 8, T * 8)
                                   for k in ("input_ids", "labels", "position_ids")])
    ws = psq.workspace_for(dev, lib.psq_process_thd_workspace(layout, B, S))
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = scal.data_ptr()

    def call(stream=stream):
        lib.psq_process_thd(layout, B, S, cu.data_ptr(), cp.data_ptr(), sp, sp + 4, sp + 8,
                            mask.data_ptr(), copies, n_c, sp + 12, ws.data_ptr(), ws.numel(),
                            stream)

    call()
    n, _, _, st = scal.cpu().tolist()
    assert st == 0, st
    algo = 16 * B * P + 48 * T + T + 8 * (n + 1) + 16
    return call, T, algo, {"workload": "thd_tables", "B": B, "S": S, "P": P, "num_seqs": n}, \
        (t, outs, cu, cp, mask, scal, ws)


def setup_pack(torch, psq, lib, synth, dev):
    w = synth.pack_sources()
    C, q = w["capacity"], w["q"]
    N = w["real_len"].size
    P = w["pack_start"].size - 1
    src = torch.from_numpy(w["src"]).to(dev)
    off = torch.from_numpy(w["src_off"]).to(dev)
    rl = torch.from_numpy(w["real_len"]).to(dev)
    ps = torch.from_numpy(w["pack_start"]).to(dev)
    packed = torch.empty((P, C), dtype=torch.int64, device=dev)
    tm = torch.empty((P, C), dtype=torch.uint8, device=dev)
    cu = torch.empty(N + P, dtype=torch.int32, device=dev)
    cp = torch.empty(N + P, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, lib.psq_pack_rows_workspace(N, P, C))
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(stream=stream):
        lib.psq_pack_rows(src.data_ptr(), src.numel(), off.data_ptr(), rl.data_ptr(), N, q,
                          None, ps.data_ptr(), P, C, 1, 0, packed.data_ptr(), tm.data_ptr(),
                          cu.data_ptr(), cp.data_ptr(), st.data_ptr(), ws.data_ptr(),
                          ws.numel(), stream)

    call()
    assert int(st.item()) == 0
    real = int(w["real_len"].sum())
    algo = 8 * real + 8 * N + 4 * N + 8 * (P + 1) + 9 * P * C + 8 * (N + P) + 4
    info = {"workload": "pack_sources", "N": N, "P": P, "capacity": C, "pad_to": q,
            "real_tokens": real}
    return call, P * C, algo, info, (src, off, rl, ps, packed, tm, cu, cp, st, ws)


def setup_split(torch, psq, lib, synth, dev, G=4):
    """Workload 3 through split_batch_into_thd_chunks with G row groups."""
    w = synth.thd_tables()
    S = w["S"]
    B, P = w["seq_lens"].shape
    T = B * S
    t = {k: torch.from_numpy(w[k]).to(dev) for k in
         ("input_ids", "labels", "position_ids", "seq_lens", "seq_lens_padded")}
    outs = {k: torch.empty(T, dtype=torch.int64, device=dev) for k in ("input_ids", "labels", "position_ids")}
    cap = G * (B // G * P + 1)
    cu = torch.empty(cap, dtype=torch.int32, device=dev)
    cp = torch.empty(cap, dtype=torch.int32, device=dev)
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    per = torch.zeros((3, G), dtype=torch.int32, device=dev)
    scal = torch.zeros(2, dtype=torch.int32, device=dev)
    layout = lib.make_layout(lib.LAYOUT_SEQ_LENS, t["seq_lens"].data_ptr(),
                             t["seq_lens_padded"].data_ptr(), lib.I64, P, -1000)
    copies, n_c = lib.make_copies([(t[k].data_ptr(), outs[k].data_ptr(), 1, T * 8, T * 8)
                                   for k in ("input_ids", "labels", "position_ids")])
    ws = psq.workspace_for(dev, lib.psq_split_thd_workspace(layout, B, S, G))
    stream = torch.cuda.current_stream(dev).cuda_stream
    pp, sp = per.data_ptr(), scal.data_ptr()

    def call(stream=stream):
        lib.psq_split_thd(layout, B, S, G, cu.data_ptr(), cp.data_ptr(), sp, pp, pp + 4 * G,
                          pp + 8 * G, mask.data_ptr(), copies, n_c, sp + 4, ws.data_ptr(),
                          ws.numel(), stream)

    call()
    width, st = scal.cpu().tolist()
    assert st == 0, st
    algo = 16 * B * P + 48 * T + T + 8 * G * width + 12 * G + 8
    info = {"workload": f"thd_tables split into {G} row groups", "B": B, "S": S, "P": P,
            "num_chunks": G, "cu_width": width}
    return call, T, algo, info, (t, outs, cu, cp, mask, per, scal, ws)


def setup_padids(torch, psq, lib, synth, dev):
    """The metadata-free padding mask of a 131072-id stream with a pad tail."""
    w = synth.pad_tail_stream()
    ids = torch.from_numpy(w["input_ids"]).to(dev)
    T = ids.numel()
    mask = torch.empty(T, dtype=torch.bool, device=dev)
    scal = torch.zeros(2, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, lib.psq_padding_mask_from_token_ids_workspace(T))
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = scal.data_ptr()

    def call(stream=stream):
        lib.psq_padding_mask_from_token_ids(ids.data_ptr(), lib.I64, T, w["pad_id"],
                                            mask.data_ptr(), sp, sp + 4, ws.data_ptr(),
                                            ws.numel(), stream)

    call()
    nc, st = scal.cpu().tolist()
    assert st == 0 and nc == T - w["tail"], (nc, st)
    algo = 8 * T + T + 8
    info = {"workload": "pad_tail_stream", "T": T, "tail": w["tail"]}
    return call, T, algo, info, (ids, mask, scal, ws)


def setup_rect(torch, psq, lib, synth, dev):
    """Trainer packs: a 256-row padded rectangle squeezed into token-budget bins."""
    w = synth.trainer_rectangle()
    rows_np, rl_np, bins, q = w["rows"], w["real_len"], w["bins"], w["q"]
    N, W = rows_np.shape
    P = len(bins)
    C = w["width"]              # chosen by the host packer with the bins
    members = [i for b in bins for i in b]
    order = torch.zeros(N, dtype=torch.int32)
    order[: len(members)] = torch.tensor(members, dtype=torch.int32)
    starts = torch.zeros(P + 1, dtype=torch.int64)
    starts[1:] = torch.tensor([len(b) for b in bins]).cumsum(0)
    rows = torch.from_numpy(rows_np).to(dev)
    rl = torch.from_numpy(rl_np).to(dev)
    order, starts = order.to(dev), starts.to(dev)
    packed = torch.empty((P, C), dtype=torch.int64, device=dev)
    tm = torch.empty((P, C), dtype=torch.uint8, device=dev)
    cu = torch.empty(N + P, dtype=torch.int32, device=dev)
    cp = torch.empty(N + P, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = psq.workspace_for(dev, lib.psq_pack_rows_workspace(N, P, C))
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(stream=stream):
        lib.psq_pack_padded_rows(rows.data_ptr(), W, rl.data_ptr(), N, q, order.data_ptr(),
                                 starts.data_ptr(), P, C, 0, 0, packed.data_ptr(), tm.data_ptr(),
                                 cu.data_ptr(), cp.data_ptr(), st.data_ptr(), ws.data_ptr(),
                                 ws.numel(), stream)

    call()
    assert int(st.item()) == 0
    real = int(rl_np.sum())
    algo = 8 * real + 4 * N + 4 * N + 8 * (P + 1) + 9 * P * C + 8 * (N + P) + 4
    info = {"workload": "trainer_rectangle", "N": N, "W": W, "bins": P, "width": C,
            "pad_to": q, "real_tokens": real}
    return call, P * C, algo, info, (rows, rl, order, starts, packed, tm, cu, cp, st, ws)


def launch_floor(torch, lib, dev, iters):
    """The library's smallest launch (psq_workspace_init of 256 bytes: one
    one-wave fill workgroup) timed like the latency-bound workloads: the floor
    under their per-call times."""
    buf = torch.empty(256, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(stream=stream):
        lib.psq_workspace_init(buf.data_ptr(), buf.numel(), stream)

    for _ in range(5):
        call()
    m, _, med = measure(torch, call, iters)
    return {"what": "psq_workspace_init of 256 bytes (one fill workgroup) through the ctypes "
                    "binding", "us_median": round(med * 1e3, 2), "us_mean": round(m * 1e3, 2),
            "us_back_to_back": round(back_to_back_ms(torch, call, iters) * 1e3, 2),
            "us_in_graph": round(graph_ms(torch, call, 20, 5) * 1e3, 2)}


def graph_ms(torch, call, calls_per_graph, replays):
    """ms per call when `calls_per_graph` calls are captured in one HIP graph
    and the graph is replayed: the launches are submitted as one graph, so
    the per-call launch cost of the isolated and back-to-back timings mostly
    goes away.  The outputs of the last replay are the ones checked against
    the oracle afterwards."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(calls_per_graph):
            call(cs)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(torch.cuda.current_stream())
    for _ in range(replays):
        g.replay()
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (replays * calls_per_graph)
    del g
    return ms


def back_to_back_ms(torch, call, iters):
    """ms per call of `iters` calls enqueued back to back between one pair of
    HIP events: the rate of a stream of calls, where each launch overlaps the
    previous call's execution instead of waiting for the host."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(torch.cuda.current_stream())
    for _ in range(iters):
        call()
    b.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def measure(torch, call, iters, flush=None):
    """(mean, min, median) ms of `iters` launches, HIP events on the launch stream."""
    timer = Timer(torch)
    for _ in range(iters):
        if flush is not None:
            flush()
        with timer:
            call()
    m, mn = timer.mean_ms()
    return m, mn, timer.median_ms()


# ---------------------------------------------------------------------------
# parity in the same run: the outputs of the last timed call against digests
# of the CPU oracle's outputs on the same seeded inputs, stored by
# tests/golden/make_digests.py (every output is an integer or a byte copy)
# ---------------------------------------------------------------------------

DIGESTS = os.path.join(ROOT, "tests", "golden", "workload_digests.json")


def _sha(t, np_dtype) -> str:
    import numpy as np
    a = t.cpu().numpy() if hasattr(t, "cpu") else t
    return hashlib.sha256(np.ascontiguousarray(a, dtype=np_dtype).tobytes()).hexdigest()


def _eq(got, want, what):
    if got != want:
        raise AssertionError(f"parity: {what} differs from the oracle's ({got!r} != {want!r})")


def check_outputs(torch, name, keep):
    import numpy as np
    with open(DIGESTS) as f:
        want = json.load(f)[name]
    i32, u8, i64 = np.int32, np.uint8, np.int64
    if name in ("doc_map_small", "doc_map_medium"):
        doc, cu, scal, _ = keep
        n, mx = int(scal[0].item()), int(scal[1].item())
        _eq((n, mx), (want["num_segments"], want["max_seqlen"]), "num_segments / max_seqlen")
        _eq(_sha(cu[: n + 1], i32), want["cu_seqlens"], "cu_seqlens")
    elif name == "thd_tables":
        t, outs, cu, cp, mask, scal, _ = keep
        n, mx, pb, st = scal.cpu().tolist()
        _eq((st, n, mx, pb), (want["status"], want["num_seqs"], want["max_seqlen"],
                              want["pad_between_seqs"]), "scalars")
        _eq(_sha(cu[: n + 1], i32), want["cu_seqlens"], "cu_seqlens")
        _eq(_sha(cp[: n + 1], i32), want["cu_seqlens_padded"], "cu_seqlens_padded")
        _eq(_sha(mask.view(torch.uint8), u8), want["padding_mask"], "padding_mask")
        for k, o in outs.items():
            _eq(_sha(o.view(torch.uint8), u8), want[k], k)
    elif name == "thd_split_4":
        t, outs, cu, cp, mask, per, scal, _ = keep
        G = per.shape[1]
        width, st = scal.cpu().tolist()
        _eq((st, width), (want["status"], want["cu_width"]), "status / cu_width")
        _eq(_sha(cu[: G * width], i32), want["cu_seqlens"], "cu_seqlens")
        _eq(_sha(cp[: G * width], i32), want["cu_seqlens_padded"], "cu_seqlens_padded")
        _eq(_sha(per, i32), want["per_chunk"], "per-chunk scalars")
        _eq(_sha(mask.view(torch.uint8), u8), want["padding_mask"], "padding_mask")
    elif name in ("pack_sources", "trainer_rectangle"):
        packed, tm, cu, cp, st = keep[-6:-1]
        used = want["csr_entries"]
        _eq(int(st.item()), want["status"], "status")
        _eq(_sha(packed, i64), want["packed"], "packed")
        _eq(_sha(tm, u8), want["token_mask"], "token_mask")
        _eq(_sha(cu[:used], i32), want["cu_seqlens"], "cu_seqlens")
        _eq(_sha(cp[:used], i32), want["cu_seqlens_padded"], "cu_seqlens_padded")
    elif name == "pad_tail_stream":
        ids, mask, scal, _ = keep
        nc, st = scal.cpu().tolist()
        _eq((nc, st), (want["num_content"], want["status"]), "num_content / status")
        _eq(_sha(mask.view(torch.uint8), u8), want["padding_mask"], "padding_mask")
    elif name == "stage_embedding":
        out_h, out_p, cu, cp, mask, scal, _ = keep["out"]
        n, mx, pb, st = scal.cpu().tolist()
        _eq((n, mx, pb, st), (want["num_segments"], want["max_seqlen"], 0, 0), "scalars")
        _eq(_sha(cu[: n + 1], i32), want["cu_seqlens"], "cu_seqlens")
        _eq(_sha(cp[: n + 1], i32), want["cu_seqlens"], "cu_seqlens_padded")
        _eq(_sha(mask.view(torch.uint8), u8), want["padding_mask"], "padding_mask")
        _eq(_sha(out_p.view(torch.uint8), u8), want["position_ids"], "position_ids")
        # the 8 GiB hidden copy is an identity: compared with its input on the
        # device in 64 MiB slices
        h = keep["hidden"].view(-1, out_h.shape[1])
        for r0 in range(0, h.shape[0], 8192):
            if not torch.equal(out_h[r0:r0 + 8192].view(torch.int16), h[r0:r0 + 8192].view(torch.int16)):
                raise AssertionError("parity: hidden differs from its input")
    return "bit-exact"


def library_copy_ceiling(torch, psq, lib, dev, nbytes=4 << 30):
    """The library's own collapse copy of 4 GiB (one-wave 1 KiB workgroups,
    behind a one-token map: psq_process_thd with one copy), timed like the
    stage step: the practical copy ceiling for this traffic on the chip."""
    call, keep = setup_calibration_copy(torch, psq, lib, dev, nbytes)
    call()
    timer = Timer(torch)
    for _ in range(10):
        with timer:
            call()
    m, mn = timer.mean_ms()
    del keep
    return {"what": "the library's one-wave collapse copy of 4 GiB (psq_process_thd, one-token "
                    "map plus one copy; the map's one workgroup is inside the timed region)",
            "gbs_mean": round(2 * nbytes / (m * 1e-3) / 1e9, 1),
            "gbs_best": round(2 * nbytes / (mn * 1e-3) / 1e9, 1)}


def copy_ceiling(torch, dev, nbytes=4 << 30):
    """A device-to-device hipMemcpyAsync (torch copy_ of contiguous tensors) of
    4 GiB: context for the collapse copy's rate."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    timer = Timer(torch)
    for _ in range(10):
        with timer:
            dst.copy_(src)
    m, mn = timer.mean_ms()
    del src, dst
    return {"what": "hipMemcpyAsync device to device, 4 GiB (torch copy_)",
            "gbs_mean": round(2 * nbytes / (m * 1e-3) / 1e9, 1),
            "gbs_best": round(2 * nbytes / (mn * 1e-3) / 1e9, 1)}


def host_cpu():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count()}


def setup_calibration_copy(torch, psq, lib, dev, nbytes=1 << 30):
    """A plain device copy of known size (the collapse path with a one-token
    map): its HBM counters calibrate the counters of the other kernels."""
    src = torch.empty(nbytes // 8, dtype=torch.int64, device=dev).random_()
    dst = torch.empty_like(src)
    doc = torch.ones((1, 1), dtype=torch.int32, device=dev)
    cu = torch.empty(2, dtype=torch.int32, device=dev)
    scal = torch.zeros(4, dtype=torch.int32, device=dev)
    layout = lib.make_layout(lib.LAYOUT_DOC_IDS, doc_ids=doc.data_ptr(), doc_dtype=lib.I32)
    copies, n_c = lib.make_copies([(src.data_ptr(), dst.data_ptr(), 1, nbytes, nbytes)])
    ws = psq.workspace_for(dev, lib.psq_process_thd_workspace(layout, 1, 1))
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp = scal.data_ptr()

    def call(stream=stream):
        lib.psq_process_thd(layout, 1, 1, cu.data_ptr(), None, sp, sp + 4, sp + 8, None, copies,
                            n_c, sp + 12, ws.data_ptr(), ws.numel(), stream)

    return call, (src, dst, doc, cu, scal, ws)


def profile_launches(torch, psq, lib, synth, dev, n, info_path=None):
    """Launch each workload n times (plus the calibration copy) for a
    counter run; prints what ran, in launch order.  With ``info_path``, writes
    each workload's algorithmic bytes there (the stage step also split into
    its collapse copy and its map)."""
    # counter calibration on kernels this library did not write: torch's
    # zero_ of a 1 GiB int64 tensor writes 1 GiB once, and torch's sum over
    # it reads 1 GiB once
    big = torch.empty(1 << 27, dtype=torch.int64, device=dev)
    for _ in range(n):
        big.zero_()
    torch.cuda.synchronize()
    for _ in range(n):
        big.sum()
    torch.cuda.synchronize()
    print(f"[profile] torch zero_ and sum over 1 GiB: {n} launches each", file=sys.stderr,
          flush=True)
    del big
    runs = [("calibration_copy_1GiB",
             lambda: (lambda c: (c[0], None, 1 << 31, None, c[1]))(
                 setup_calibration_copy(torch, psq, lib, dev)))]
    for name, setup in (("stage_embedding", lambda: setup_stage_embedding(torch, psq, lib, synth, dev)),
                        ("pack_sources", lambda: setup_pack(torch, psq, lib, synth, dev)),
                        ("thd_tables", lambda: setup_thd(torch, psq, lib, synth, dev)),
                        ("doc_map_medium", lambda: setup_doc_map(torch, psq, lib, synth, dev, 2)),
                        ("thd_split_4", lambda: setup_split(torch, psq, lib, synth, dev)),
                        ("pad_tail_stream", lambda: setup_padids(torch, psq, lib, synth, dev)),
                        ("trainer_rectangle", lambda: setup_rect(torch, psq, lib, synth, dev))):
        runs.append((name, setup))
    algo = {}
    for name, setup in runs:
        call, _, algo[name], info, keep = setup()
        if name == "stage_embedding":
            T, H = info["B"] * info["S"], info["H"]
            algo["stage_copy"] = 4 * T * H + 16 * T     # bf16 hidden and int64 positions, read + write
            algo["stage_map"] = algo[name] - algo["stage_copy"]
        torch.cuda.synchronize()
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        print(f"[profile] {name}: {n} launches", file=sys.stderr, flush=True)
        del keep
    if info_path:
        with open(info_path, "w") as f:
            json.dump(algo, f, indent=1)


def roofline(algo_bytes, mean_ms, traffic=None):
    gbs = algo_bytes / (mean_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


def oracle_workload(name, synth):
    """The CPU oracle on a per-config workload: (run, description).  ``run``
    makes the computation of the GPU call on the same seeded inputs (drawn
    again from the same generators)."""
    import oracle
    if name in ("doc_map_small", "doc_map_medium"):
        d = synth.doc_map_small() if name == "doc_map_small" else synth.doc_map_medium()
        return (lambda: oracle.doc_segments(d, want_mask=False)), \
            f"segmentation of the whole map {list(d.shape)}"
    if name in ("thd_tables", "thd_split_4"):
        w = synth.thd_tables()
        L, Lp, S = w["seq_lens"], w["seq_lens_padded"], w["S"]
        keys = ("input_ids", "labels", "position_ids")

        def run():
            if name == "thd_tables":
                oracle.thd_tables(L, Lp, S)
            else:
                oracle.split_thd(L, Lp, S, 4)
            for k in keys:
                oracle.copy_rows(w[k], 1, w[k].nbytes, w[k].nbytes)
        what = "metadata and mask" if name == "thd_tables" else "metadata and mask in 4 row groups"
        return run, f"the whole batch {list(L.shape)}, S={S}: {what}, three int64 collapses"
    if name == "pack_sources":
        w = synth.pack_sources()
        return (lambda: oracle.pack(w["src"], w["src_off"], w["real_len"], w["q"],
                                    w["pack_start"], w["capacity"], fold=True)), \
            f"all {w['real_len'].size} sources into {w['pack_start'].size - 1} packs"
    if name == "pad_tail_stream":
        w = synth.pad_tail_stream()
        return (lambda: oracle.pad_mask_from_ids(w["input_ids"], w["pad_id"])), \
            f"the whole stream of {w['input_ids'].size} ids"
    if name == "trainer_rectangle":
        w = synth.trainer_rectangle()
        return (lambda: oracle.pack_rect(w["rows"], w["real_len"], w["q"], w["bins"],
                                         width=w["width"])), \
            f"all {w['real_len'].size} rows into {len(w['bins'])} bins"
    raise KeyError(name)


def time_oracle(run, reps=3):
    """One warm-up run, then the median of ``reps`` runs (seconds)."""
    run()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2]


def per_config_cpu_baseline(name, synth, tokens, gpu_ms, host):
    run, what = oracle_workload(name, synth)
    t = time_oracle(run)
    return {"value": round(tokens / t / 1e9, 6), "unit": "Gtok/s", "seconds": round(t, 6),
            "cores": 1, "kind": "oracle",
            "sample": f"the whole workload on the same seeded inputs ({what}), one warm-up then "
                      f"the median of 3, single-threaded C at -O2",
            "gpu_speedup": round(t / (gpu_ms * 1e-3), 1), "host": host}


def cpu_baseline(torch, keep):
    """The oracle on the whole stage-embedding workload (all 32 rows: the map,
    the mask, and both collapses, 8 GiB of bf16 hidden), one warm-up then the
    median of 5 runs: about 12 s of single-threaded CPU work."""
    import numpy as np

    import oracle
    doc_np = np.ascontiguousarray(keep["host"]["doc_ids"])
    hidden = keep["hidden"]
    H = hidden.shape[2]
    host_h = hidden.view(torch.int16).cpu().numpy()
    host_p = keep["host"]["position_ids"]
    times = []
    for rep in range(6):
        t0 = time.perf_counter()
        oracle.doc_segments(doc_np)
        out_h = oracle.copy_rows(host_h, 1, host_h.nbytes, host_h.nbytes)
        oracle.copy_rows(host_p, 1, host_p.nbytes, host_p.nbytes)
        if rep > 0:                      # the first run is the warm-up
            times.append(time.perf_counter() - t0)
        del out_h
    t = sorted(times)[len(times) // 2]
    tokens = doc_np.size
    return {"value": round(tokens / t / 1e9, 6), "unit": "Gtok/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload: {doc_np.shape[0]} rows ({tokens} tokens, "
                      f"{tokens * H * 2 >> 30} GiB of bf16 hidden): segmentation + mask + both "
                      f"collapses, one warm-up then the median of 5, single-threaded C at -O2",
            "seconds": round(t, 3), "seconds_total": round(sum(times), 1), "host": host_cpu()}


WORKLOAD_OF = {
    "k_copies": "collapse copies",
    "k_pack_rows": "pack_sources: 65536 sources -> 16384-slot packs; trainer_rectangle: "
                   "256 rows -> token-budget bins",
    "k_thd_small": "thd_tables: 16 x 64 tables, S=8192, three int64 collapses "
                   "(whole batch, and split into 4 row groups)",
    "k_thd_tables_copy": "length tables above 2048 entries, with collapses",
    "k_doc_small": "document maps of 4097 .. 4194304 positions (one launch over up to 256 "
                   "tiles of 1024 to 16384 positions)",
    "k_doc_scatter": "document maps of up to 4096 positions (one workgroup), or launch 2 of "
                     "larger maps than one launch takes",
    "k_doc_reduce": "launch 1 of document maps above 4194304 positions",
    "k_pad_ids": "pad_tail_stream: 131072 int64 ids with a pad tail",
    "k_zero_fill": "workspace zero fill (once per workspace)",
}


# (kernel, grid size in threads) -> workload, for kernels that serve several
GRID_LABEL = {
    ("k_pack_rows", "4263296"): "pack_sources: 65536 sources -> 3506 packs of 16384 slots",
    ("k_pack_rows", "61440"): "trainer_rectangle: 256 rows -> 15 token-budget bins",
    ("k_doc_scatter", "256"): "doc_map_small [4,64] (and the one-token maps of the copy "
                              "calibrations and ceiling)",
    ("k_doc_small", "8192"): "doc_map_medium [8,4096] (32 tiles of 1024 positions)",
    ("k_doc_small", "65536"): "stage_embedding step, launch 1: doc map [32,32768] (256 tiles "
                              "of 4096 positions) -> cu_seqlens, max_seqlen, mask",
    ("k_copies", "537395200"): "stage_embedding step, launch 2: bf16 [32,32768,4096] + int64 "
                               "positions collapse (8 GiB + 8 MiB)",
    ("k_copies", "67108864"): "1 GiB calibration copy (counter runs only)",
    ("k_copies", "268435456"): "4 GiB one-wave copy: the library's copy ceiling",
    ("k_zero_fill", "64"): "launch floor: psq_workspace_init of 256 bytes (isolated, back to "
                           "back and in a HIP graph)",
}


def summarize_trace(stats_csv: str, out_md: str, command: str) -> None:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: the
    kernel_stats.csv totals, split per launch grid with the sibling
    kernel_trace.csv (one kernel can serve several workloads)."""
    import csv
    import statistics
    trace_csv = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    lines = ["# Kernel trace: " + os.path.basename(out_md)[:-3], "",
             "Command (on an MI355X, from the repository root):", "", "```", command, "```", "",
             "| kernel | grid (threads) | workload | calls | avg us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        if "psq::" not in r["Kernel_Name"]:
            continue
        short = kernel_short_name(r["Kernel_Name"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault((short, r["Grid_Size_X"]), []).append(dur)
    for (short, grid), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        base = short.split("<")[0].replace("psq::", "")
        label = GRID_LABEL.get((base, grid), WORKLOAD_OF.get(base, ""))
        lines.append(f"| `{short}` | {grid} | {label} | {len(v)} | {statistics.mean(v):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    lines += ["", "Per-kernel totals from kernel_stats.csv:", "",
              "| kernel | calls | avg us |", "|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        if "psq::" in r["Name"]:
            lines.append(f"| `{kernel_short_name(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, launch_info=args.launch_info)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this path has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import varlen_attention_metadata_amd as psq
    from varlen_attention_metadata_amd import _lib as lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_launches > 0:
        profile_launches(torch, psq, lib, synth, dev, args.profile_launches, args.launch_info)
        return

    call, tokens, algo, info, keep = setup_stage_embedding(torch, psq, lib, synth, dev)
    print(f"[bench] stage_embedding ready: {algo / 1e9:.2f} GB per step", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        with timer:
            call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3
    k_mean, k_min = timer.mean_ms()
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, kernel {k_mean:.3f} ms",
          file=sys.stderr, flush=True)
    parity = check_outputs(torch, "stage_embedding", keep) if not args.no_check else "not checked"
    print(f"[bench] stage_embedding parity: {parity}", file=sys.stderr, flush=True)

    traffic = None
    tr = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash():
            traffic = tr.get("bytes_per_launch")

    def workload_traffic(name):
        """Counter bytes per launch of a per-config workload, or None once its
        kernel's sources differ from those the counters were taken on."""
        w = tr.get("workloads", {}).get(name)
        if w is None or name not in WORKLOAD_COUNTERS:
            return None
        return w["bytes_per_launch"] if w["source_hash"] == source_hash(WORKLOAD_COUNTERS[name][1]) else None

    result = {
        "metric": METRIC,
        "value": round(tokens / (ms_per_step * 1e-3) / 1e9, 4),
        "unit": "Gtok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32 map; bf16 hidden and int64 positions copied bitwise",
        "data": "synthetic (seeded generators; bf16 hidden N(0,1) drawn on the device)",
        "parity": parity,
        "config": dict(info, **{"algorithmic_bytes_per_step": algo,
                                "hbm_gbs_per_step": round(algo / (ms_per_step * 1e-3) / 1e9, 1)}),
        "roofline": dict(roofline(algo, k_mean, traffic),
                         kernel="k_doc_small<int, 4> + k_copies<u32x4,true>: one psq_process_thd "
                                "call, the metadata launch then the collapse copy (HIP events "
                                "bracket both)",
                         kernel_ms_mean=round(k_mean, 4), kernel_ms_median=round(timer.median_ms(), 4),
                         kernel_ms_min=round(k_min, 4)),
    }

    host = host_cpu()
    if not args.no_per_config:
        per = {}
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def flush():
            flush_buf.fill_(1)

        for name, setup, do_flush in (
                ("doc_map_small", lambda: setup_doc_map(torch, psq, lib, synth, dev, 1), False),
                ("doc_map_medium", lambda: setup_doc_map(torch, psq, lib, synth, dev, 2), False),
                ("thd_tables", lambda: setup_thd(torch, psq, lib, synth, dev), False),
                ("pack_sources", lambda: setup_pack(torch, psq, lib, synth, dev), True),
                ("thd_split_4", lambda: setup_split(torch, psq, lib, synth, dev), False),
                ("pad_tail_stream", lambda: setup_padids(torch, psq, lib, synth, dev), False),
                ("trainer_rectangle", lambda: setup_rect(torch, psq, lib, synth, dev), True)):
            c_call, c_tok, c_algo, c_info, c_keep = setup()
            for _ in range(5):
                c_call()
            m, mn, med = measure(torch, c_call, args.per_config_iters,
                                 flush if do_flush else None)
            b2b = None if do_flush else back_to_back_ms(torch, c_call, args.per_config_iters)
            in_graph = None if do_flush else graph_ms(torch, c_call, 20, 5)
            parity = check_outputs(torch, name, c_keep) if not args.no_check else "not checked"
            per[name] = dict(c_info, **{
                "us_mean": round(m * 1e3, 2), "us_median": round(med * 1e3, 2),
                "us_min": round(mn * 1e3, 2),
                "us_back_to_back": None if b2b is None else round(b2b * 1e3, 2),
                "us_in_graph": None if in_graph is None else round(in_graph * 1e3, 2),
                "gtok_s": round(c_tok / (m * 1e-3) / 1e9, 4), "tokens_per_call": c_tok,
                "algorithmic_bytes": c_algo, "roofline": roofline(c_algo, m, workload_traffic(name)),
                "parity": parity})
            del c_keep
            if not args.no_cpu_baseline:
                per[name]["cpu_baseline"] = per_config_cpu_baseline(name, synth, c_tok, m, host)
            print(f"[bench] {name}: {m * 1e3:.2f} us, parity {parity}"
                  + (f", oracle {per[name]['cpu_baseline']['seconds'] * 1e3:.2f} ms"
                     if "cpu_baseline" in per[name] else ""), file=sys.stderr, flush=True)
        per["stage_embedding"] = {"us_mean": round(k_mean * 1e3, 2), "gtok_s": result["value"],
                                  "roofline": roofline(algo, k_mean, traffic),
                                  "parity": result["parity"],
                                  "cpu_baseline": "the top-level cpu_baseline"}
        result["per_config"] = per
        del flush_buf
        result["copy_ceiling"] = copy_ceiling(torch, dev)
        result["copy_ceiling_library"] = library_copy_ceiling(torch, psq, lib, dev)
        result["launch_floor"] = launch_floor(torch, lib, dev, args.per_config_iters)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, keep)
        print(f"[bench] cpu baseline: {result['cpu_baseline']['seconds']} s", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
