"""Benchmark of the token-tree attention + verification path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
tree attention -> stochastic tree verification -> accepted-path KV compaction
(the ancestor-mask build and the split-K merge run inside the attention kernel,
row statistics / decisions / path selection inside the verification kernel).

Prints ONE JSON line.  `value` = tree nodes verified per second over the timed
steps (sum of n_nodes over the batch / seconds per step), inputs resident in
HBM.  Every step reads a different copy of the inputs (rotating through at least
1 GiB) so the 256 MB Infinity Cache cannot serve repeated reads.

Per-kernel durations come from HIP events recorded on the stream the kernels run
on (torch's current stream), averaged over back-to-back calls on rotating copies.
The CPU oracle is timed on a bounded sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tree nodes verified/sec + tree-attn HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
# dense compute peaks, vendor figures: bf16 on MFMA; float32 attention runs on the vector ALUs
COMPUTE_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama8b",
                    choices=["tiny", "llama8b", "ragged", "chain", "llama70b_share"])
    ap.add_argument("--kernel-reps", type=int, default=100, help="back-to-back calls per kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bound on the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-construction", action="store_true", help="skip the tree-construction timings")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--table-tokens", type=int, default=0,
                    help="size every request's block table for this many tokens of context (entries past "
                         "the request's blocks are -1); 0: exactly the blocks the request uses")
    ap.add_argument("--accept-seeds", type=int, default=16,
                    help="workload seeds whose stochastic verification gives the acceptance statistics")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed step")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one elementwise copy of this many MiB (a reference "
                         "kernel of known traffic for hardware byte counters)")
    ap.add_argument("--budget-table", action="store_true",
                    help="instead of the step: measure step latency per (batch size, tree shape) at this "
                         "workload's layer shape and print the goodput tree-size table")
    ap.add_argument("--budget-out", default=None, help="also write the table as markdown to this path")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="no GPU work: turn a rocprofv3 --pmc run of this script with SQ_VALU_MFMA_BUSY_CYCLES, "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_BUSY_CU_CYCLES and GRBM_GUI_ACTIVE into "
                         "profiles/mfma_<workload>.md")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, both with --calibrate-copy-mib) into profiles/traffic_*.json")
    return ap.parse_args()


def gated_us_per_call(call, reps: int, cyc_per_s: float) -> float:
    """GPU microseconds per call of `reps` back-to-back calls (call(i) enqueues call i).

    A spin kernel holds the stream while the host enqueues the calls, so that the
    events bracket GPU execution only.  The spin is sized from an untimed pass of
    the same calls; if the timed pass's enqueueing outlasts the spin (the GPU
    would then wait for the host inside the timed region), the pass is repeated
    with a longer spin, at most twice."""
    import torch
    h0 = time.perf_counter()
    for i in range(reps):
        call(i)
    spin_s = 2.0 * (time.perf_counter() - h0) + 2e-3
    torch.cuda.synchronize()
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(cyc_per_s * spin_s))
        a.record()
        h1 = time.perf_counter()
        for i in range(reps):
            call(i)
        enq_s = time.perf_counter() - h1
        b.record()
        torch.cuda.synchronize()
        if enq_s < 0.8 * spin_s:
            break
        spin_s = 3.0 * enq_s + 2e-3
    return a.elapsed_time(b) / reps * 1e3


def kernel_is(name: str, full: str) -> bool:
    """True when the profiler's kernel name `full` is kernel `name` (a whole
    identifier: merge_kernel is not tree_merge_kernel)."""
    return re.search(r"(?<![A-Za-z0-9_])" + re.escape(name) + r"(?![A-Za-z0-9_])", full) is not None


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "tree_verification_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


# kernels launched by each entry point (rocprofv3 kernel names contain these)
ENTRY_KERNELS = {
    "tree_attn": ("tree_attn_kernel",),
    "tree_verify_stochastic": ("stoch_node_kernel",),
    "tree_verify_greedy": ("greedy_argmax_kernel",),
    "kv_compact": ("compact_kernel",),
    "tree_verify_stochastic_compact": ("stoch_node_kernel",),
}
ENTRY_SOURCES = {"tree_attn": ("tree_attn.hip",), "tree_verify_stochastic": ("tree_verify.hip",),
                 "tree_verify_greedy": ("tree_verify.hip",), "kv_compact": ("kv_compact.hip", "tv_compact.h"),
                 "tree_verify_stochastic_compact": ("tree_verify.hip", "tv_compact.h")}
CALIB_KERNEL = "elementwise"


def read_counters(run_dir: str, counter: str):
    """(kernel name, value) per dispatch for one counter from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return [(k, v) for _, k, v in rows]


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, calib_mib: int):
    out = {}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_counters(d, counter)
        calib = [v for k, v in rows if CALIB_KERNEL in k]
        if not calib:
            raise SystemExit(f"no calibration kernel among the {counter} dispatches in {d}")
        scale = (calib_mib << 20) / (calib[-1] * 1024.0)   # counter KiB -> bytes
        per[counter] = {"calibration_kib": calib[-1], "bytes_per_kib": scale}
        for entry, names in ENTRY_KERNELS.items():
            first = [v for k, v in rows if kernel_is(names[0], k)]
            if not first:
                continue
            tot = sum(v for k, v in rows if any(kernel_is(nm, k) for nm in names))
            out.setdefault(entry, {})[counter] = tot * 1024.0 * scale / len(first)
            out[entry]["launches"] = len(first)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for entry, rec in out.items():
        if "FETCH_SIZE" not in rec or "WRITE_SIZE" not in rec:
            continue
        doc = {"entry_point": entry, "workload": workload, "kernels": list(ENTRY_KERNELS[entry]),
               "source_hash": source_hash(*ENTRY_SOURCES[entry]),
               "fetch_bytes_per_launch": round(rec["FETCH_SIZE"]), "write_bytes_per_launch": round(rec["WRITE_SIZE"]),
               "hbm_bytes_per_launch": round(rec["FETCH_SIZE"] + rec["WRITE_SIZE"]),
               "launches_counted": rec["launches"], "calibration": per,
               "method": "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of bench.py, each counter "
                         f"scaled by its reading for a {calib_mib} MiB elementwise copy"}
        path = os.path.join(ROOT, "profiles", f"traffic_{entry}_{workload}.json")
        json.dump(doc, open(path, "w"), indent=1)
        print(path, doc["hbm_bytes_per_launch"])


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.config, args.calibrate_copy_mib or 256)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, args.config)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from tree_verification_amd import binding as tv
    from tree_verification_amd.workloads import bf16_bits, make_workload, seed_for

    if args.budget_table:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        budget_table(args, torch.device("cuda:0"))
        return
    seed = seed_for(args.config) if args.seed is None else args.seed
    t0 = time.time()
    wl = make_workload(args.config, seed=seed)
    if args.table_tokens > 0:
        widen_table(wl, args.table_tokens)
    gen_s = time.time() - t0
    # the CPU oracle first: its worker processes are forked before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    tv.load_library()
    dev = torch.device("cuda:0")
    B, Nmax, V = wl.batch, wl.n_max, wl.vocab
    n_total = int(wl.n_nodes.sum())
    esize = 2 if wl.dtype == "bf16" else 4

    def kv(x):
        if wl.dtype == "bf16":
            return torch.from_numpy(bf16_bits(x)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    base = dict(q=kv(wl.q), k=kv(wl.k_cache), v=kv(wl.v_cache), table=i32(wl.block_table),
                pre=i32(wl.prefix_len), nn=i32(wl.n_nodes), par=i32(wl.parent), tok=i32(wl.tokens),
                tl=torch.from_numpy(wl.target_logits).to(dev), dl=torch.from_numpy(wl.draft_logits).to(dev),
                ua=torch.from_numpy(wl.u_accept).to(dev), us=torch.from_numpy(wl.u_sample).to(dev))
    copy_bytes = sum(t.numel() * t.element_size() for t in base.values())
    ncopies = max(2, math.ceil(ROTATE_BYTES / copy_bytes))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(ncopies - 1)]
    pristine_k, pristine_v = base["k"].clone(), base["v"].clone()
    for c in copies:
        c["out"] = torch.empty_like(c["q"])
        c["ast"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["path"] = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
        c["plen"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["otok"] = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
        c["vst"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["gpath"] = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
        c["gplen"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["gotok"] = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
        c["gst"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["src"] = torch.empty((B, Nmax), dtype=torch.int32, device=dev)
        c["nlen"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["cst"] = torch.empty(B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def attn(c):
        tv.tree_attn_forward(c["q"], c["k"], c["v"], c["table"], c["pre"], c["nn"], c["par"],
                             out=c["out"], status=c["ast"])

    def verify(c):
        tv.tree_verify_stochastic(c["tl"], c["dl"], c["tok"], c["par"], c["nn"], c["ua"], c["us"],
                                  path=c["path"], path_len=c["plen"], out_tokens=c["otok"], status=c["vst"])

    def greedy(c):
        tv.tree_verify_greedy(c["tl"], c["tok"], c["par"], c["nn"], path=c["gpath"], path_len=c["gplen"],
                              out_tokens=c["gotok"], status=c["gst"])

    def compact(c):
        tv.kv_compact_accepted(c["k"], c["v"], c["table"], c["pre"], c["path"], c["plen"],
                               src_pos=c["src"], new_len=c["nlen"], status=c["cst"])

    def verify_compact(c):
        tv.tree_verify_stochastic_compact(c["tl"], c["dl"], c["tok"], c["par"], c["nn"], c["ua"], c["us"],
                                          c["k"], c["v"], c["table"], c["pre"], path=c["path"],
                                          path_len=c["plen"], out_tokens=c["otok"], status=c["vst"],
                                          src_pos=c["src"], new_len=c["nlen"], kv_status=c["cst"])

    # The step: tree attention, then stochastic verification with the accepted
    # path's KV compaction (one call whose last kernel does both).  The same
    # work as three separate calls is timed beside it.
    def step(c):
        attn(c)
        verify_compact(c)

    def step_separate(c):
        attn(c)
        verify(c)
        compact(c)

    # one untimed step on copy 0, then restore its caches (compaction moved slots)
    step(copies[0])
    torch.cuda.synchronize()
    assert int(copies[0]["ast"].abs().sum()) == 0 and int(copies[0]["vst"].abs().sum()) == 0
    path0 = copies[0]["path"].cpu().numpy()
    plen0 = copies[0]["plen"].cpu().numpy()
    copies[0]["k"].copy_(pristine_k)
    copies[0]["v"].copy_(pristine_v)
    del pristine_k, pristine_v

    # ---- whole-step timing -------------------------------------------------
    # A spin kernel holds the stream while the host enqueues the timed calls, so
    # the events bracket GPU execution only (gated_us_per_call); the stream is
    # synchronised on both sides of the timed region.
    def spin_cycles_per_s():
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(20_000_000)
        b.record()
        torch.cuda.synchronize()
        return 20_000_000 / (a.elapsed_time(b) * 1e-3)

    cyc_per_s = spin_cycles_per_s()

    def time_steps(fn):
        return gated_us_per_call(lambda i: fn(copies[i % ncopies]), args.steps, cyc_per_s) * 1e-3

    def warm(fn):
        for i in range(args.warmup):
            fn(copies[i % ncopies])
        torch.cuda.synchronize()

    # The same work as three separate calls is timed first, in a second round
    # after one untimed round (the first timed loop after a short warm-up runs
    # slower while the GPU ramps up); then the step: `warmup` untimed steps and
    # exactly `steps` timed ones.
    warm(step_separate)
    time_steps(step_separate)
    ms_step_separate = time_steps(step_separate)
    warm(step)
    ms_step = time_steps(step)

    # the same step replayed as HIP graphs (one per rotating copy, captured on a
    # side stream after an eager warm-up there, so the captured calls reuse that
    # stream's prepared workspaces)
    ms_step_graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in copies:
                step(c)
        side.synchronize()
        graphs = []
        for c in copies:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(c)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % ncopies].replay()
        torch.cuda.synchronize()
        ms_step_graph = gated_us_per_call(lambda i: graphs[i % ncopies].replay(), args.steps, cyc_per_s) * 1e-3
        del graphs

    # ---- per-kernel timing (back-to-back calls on rotating copies) ----------

    def time_calls(fn, reps):
        for i in range(min(reps, 5)):
            fn(copies[i % ncopies])
        torch.cuda.synchronize()
        return gated_us_per_call(lambda i: fn(copies[i % ncopies]), reps, cyc_per_s)

    us_attn = time_calls(attn, args.kernel_reps)
    us_verify = time_calls(verify, args.kernel_reps)
    us_greedy = time_calls(greedy, args.kernel_reps)
    us_compact = time_calls(compact, args.kernel_reps)
    us_vc = time_calls(verify_compact, args.kernel_reps)

    # The practical streaming ceiling the HBM-bound kernels are compared with: a
    # device-to-device copy of 256 MiB (256 MiB read and 256 MiB written per call).
    copy_src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    copy_dst = torch.empty_like(copy_src)
    copy_dst.copy_(copy_src)
    torch.cuda.synchronize()
    us_copy = gated_us_per_call(lambda i: copy_dst.copy_(copy_src), 10, cyc_per_s)
    copy_bytes_moved = 2 * copy_src.numel() * 4
    del copy_src, copy_dst

    # ---- algorithmic bytes --------------------------------------------------
    P = wl.prefix_len.astype(np.int64)
    n = wl.n_nodes.astype(np.int64)
    H, Hkv, D = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    attn_bytes = int((2 * n.sum() * H * D + 2 * (P + n).sum() * Hkv * D) * esize)
    # prefix part: every (node, q-head) row against every prefix key (QK^T and PV)
    attn_flops = int(sum(4 * int(n[b]) * H * D * int(P[b]) for b in range(B)))
    # tree part: each node attends to its depth + 1 tree keys
    for b in range(B):
        par = wl.parent[b]
        depth = np.zeros(int(n[b]), dtype=np.int64)
        for u in range(1, int(n[b])):
            depth[u] = depth[par[u]] + 1
        attn_flops += int(4 * H * D * (depth + 1).sum())
    internal = 0
    passes = 0
    for b in range(B):
        nb = int(n[b])
        par = wl.parent[b, :nb]
        internal += len(set(int(x) for x in par[1:]))
        # residual passes realised on the accepted path: rejected siblings before
        # each accepted child, and every child of the final node
        L = int(plen0[b])
        pth = [int(x) for x in path0[b, :L]]
        for j, u in enumerate(pth):
            kids = [c for c in range(1, nb) if par[c] == u]
            passes += kids.index(pth[j + 1]) if j + 1 < L else len(kids)
    row = V * 4
    # The algorithm reads every target row and the draft row of every node with
    # children once (statistics and status checks), then both rows again for
    # each residual pass on the accepted path (a rejected sibling before each
    # accepted child, every child of the last node) and for the final draw (the
    # target row, and the draft row when the last node has children).  The
    # kernels hold the rows on chip across those passes (vocabularies up to
    # 131072), so their HBM traffic stays near the first term.
    draw_rows = 0
    for b in range(B):
        nb = int(n[b])
        L = int(plen0[b])
        last = int(path0[b, L - 1]) if L > 0 else 0
        draw_rows += 2 if any(int(wl.parent[b, c]) == last for c in range(1, nb)) else 1
    verify_first_bytes = int(n.sum() * row + internal * row)
    verify_bytes = verify_first_bytes + int((2 * passes + draw_rows) * row)
    greedy_bytes = int(n.sum() * row)
    compact_bytes = int(2 * 2 * plen0.astype(np.int64).sum() * Hkv * D * esize)

    def gbs(nbytes, us):
        return nbytes / (us * 1e-6) / 1e9

    kernels = {
        "tree_attn": {"us": us_attn, "bytes": attn_bytes, "GBps": gbs(attn_bytes, us_attn),
                      "TFLOPs": attn_flops / (us_attn * 1e-6) / 1e12},
        "tree_verify_stochastic": {"us": us_verify, "bytes": verify_bytes, "GBps": gbs(verify_bytes, us_verify)},
        "kv_compact": {"us": us_compact, "bytes": compact_bytes, "GBps": gbs(compact_bytes, us_compact)},
        "tree_verify_stochastic_compact": {"us": us_vc, "bytes": verify_bytes + compact_bytes,
                                           "GBps": gbs(verify_bytes + compact_bytes, us_vc)},
    }
    copy_gbs = gbs(copy_bytes_moved, us_copy)
    for k in kernels.values():
        k["frac_hbm"] = k["GBps"] / HBM_PEAK_GBS
        k["frac_copy"] = k["GBps"] / copy_gbs
    # the dominant kernel among the per-row entry points (the fused call is both rows)
    dominant = max((k for k in kernels if k != "tree_verify_stochastic_compact"), key=lambda k: kernels[k]["us"])

    def roofline(name):
        k = kernels[name]
        traffic = traffic_record(name, args.config, source_hash(*ENTRY_SOURCES[name]))
        peak_tf = COMPUTE_PEAK_TFLOPS.get(wl.dtype, COMPUTE_PEAK_TFLOPS["fp32"])
        if name == "tree_attn" and attn_flops / attn_bytes > peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
            # arithmetic intensity past the ridge point: bound by the matrix cores
            return {"kernel": name, "bound": "mfma" if wl.dtype == "bf16" else "alu",
                    "achieved": round(k["TFLOPs"], 1), "peak": peak_tf, "unit": "TFLOP/s",
                    "frac": round(k["TFLOPs"] / peak_tf, 4), "traffic": traffic,
                    "algorithmic_flops_per_launch": attn_flops, "algorithmic_bytes_per_launch": k["bytes"],
                    "avg_launch_us": round(k["us"], 3)}
        return {"kernel": name, "bound": "hbm", "achieved": round(k["GBps"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(k["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": k["bytes"], "avg_launch_us": round(k["us"], 3)}

    if args.calibrate_copy_mib > 0:
        # a plain elementwise kernel that reads and writes exactly this many bytes
        nf = (args.calibrate_copy_mib << 20) // 4
        src_buf = torch.ones(nf, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        torch.mul(src_buf, 1.0, out=dst_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    # tree construction on the GPU, timed before any host-side oracle work
    constr = None if args.no_construction else bench_construction(args, dev, cyc_per_s)

    accept = acceptance_stats(args, dev, tv, make_workload)

    value = n_total / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step": "tree_attn_forward + tree_verify_stochastic_compact",
        "ms_per_step_separate_calls": ms_step_separate,
        "ms_per_step_graph": ms_step_graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": args.config, "batch": B, "tree_nodes": n_total, "n_max": Nmax,
                   "prefix_len_total": int(P.sum()), "q_heads": H, "kv_heads": Hkv, "head_dim": D,
                   "vocab": V, "kv_dtype": wl.dtype, "verify": "stochastic", "seed": seed,
                   "table_tokens": int(wl.max_blocks * wl.block_size),
                   "rotating_copies": ncopies, "bytes_per_copy": copy_bytes},
        "roofline": roofline(dominant),
        "tree_attn_roofline": roofline("tree_attn"),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                    for k, d in kernels.items()},
        "greedy": {"us_per_call": round(us_greedy, 3), "bytes": greedy_bytes,
                   "GBps": round(gbs(greedy_bytes, us_greedy), 1),
                   "frac_copy": round(gbs(greedy_bytes, us_greedy) / copy_gbs, 4),
                   "nodes_per_s": n_total / (us_greedy * 1e-6)},
        "copy_ceiling": {"GBps": round(copy_gbs, 1), "us_per_call": round(us_copy, 3),
                         "bytes_per_call": copy_bytes_moved,
                         "what": "device-to-device copy of 256 MiB (read and write), timed like the kernels"},
        "accepted_mean": float(plen0.mean() - 1),
        "rejection_passes_on_path": passes,
        "verify_bytes_first_reads": verify_first_bytes,
        "acceptance": accept,
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 2),
    }
    if constr is not None:
        if not args.no_cpu_baseline:
            construction_oracle(constr)
        line["construction"] = {k: v for k, v in constr.items() if not k.startswith("_")}
        if "expand" in line["construction"]:
            line["construction"]["expand"]["frac_copy"] = round(line["construction"]["expand"]["GBps"] / copy_gbs, 4)
        line["budget"] = constr.pop("_budget")
    print(json.dumps(line), flush=True)


# Token-tree construction, measured beside the step (not part of `value`):
#   expand: one level of a <3, 2, 1, 1> schedule at a Llama-3 vocabulary, a batch
#           of 16 requests with 6 frontier nodes each (k = 1), i.e. 96 draft rows
#           of 128256 logits read per call;
#   merge:  4 draft models' 8-token guesses per request, a batch of 64 requests.
EXPAND_SHAPE = dict(batch=16, f_max=6, vocab=128256, k=1, n_max=1024, n0=10)
MERGE_SHAPE = dict(batch=64, n_cand=4, max_len=8, vocab=128256, n_max=64)
#   pool:   speculative blocks of 64-node trees after 4096-token prefixes in 16-token
#           blocks, a batch of 64: allocation of 4 blocks per request, then release
#           of the 3 past a 3-token accepted path.
POOL_SHAPE = dict(batch=64, prefix=4096, nodes=64, accepted=3, block=16)
#   budget: expected acceptance length of 256 trees of up to 128 nodes.
BUDGET_SHAPE = dict(batch=256, n_max=128)


def bench_construction(args, dev, cyc_per_s):
    import torch
    from tree_verification_amd import binding as tv
    from tree_verification_amd.workloads import make_candidates, make_expand_rows

    def timed(fns, reps):
        """GPU microseconds per call of back-to-back calls (rotating over fns), behind a
        spin kernel that holds the stream while the host enqueues them."""
        for f in fns[:2]:
            f()
        torch.cuda.synchronize()
        return gated_us_per_call(lambda i: fns[i % len(fns)](), reps, cyc_per_s)

    out = {}
    e = EXPAND_SHAPE
    B, F, V, k, n_max, n0 = e["batch"], e["f_max"], e["vocab"], e["k"], e["n_max"], e["n0"]
    seed = 4242
    rows_host = make_expand_rows(B, F, V, seed)
    rng = np.random.default_rng(seed)
    front_host = rng.integers(0, n0, size=(B, F)).astype(np.int32)
    rows0 = torch.from_numpy(rows_host).to(dev)
    ncp = max(2, math.ceil(ROTATE_BYTES / (rows0.numel() * 4)))
    sets = []
    for i in range(ncp):
        sets.append(dict(rows=rows0 if i == 0 else rows0.clone(),
                         fr=torch.from_numpy(front_host).to(dev),
                         nf=torch.full((B,), F, dtype=torch.int32, device=dev),
                         tok=torch.zeros((B, n_max), dtype=torch.int32, device=dev),
                         par=torch.full((B, n_max), -1, dtype=torch.int32, device=dev),
                         nn=torch.full((B,), n0, dtype=torch.int32, device=dev),
                         nfo=torch.empty((B, F * k), dtype=torch.int32, device=dev),
                         nnew=torch.empty(B, dtype=torch.int32, device=dev),
                         st=torch.empty(B, dtype=torch.int32, device=dev)))

    def expand_fn(c):
        return lambda: tv.tree_expand_topk(c["rows"], c["fr"], c["nf"], c["tok"], c["par"], c["nn"], k,
                                           new_frontier=c["nfo"], n_new=c["nnew"], status=c["st"])

    reps = max(args.kernel_reps, 20)
    # every call appends F * k nodes per request: reset the counts so that no call overflows
    # (timed() makes up to four passes of `reps` calls plus two warm-up calls)
    us_exp = timed([expand_fn(c) for c in sets], min(reps, ((n_max - n0) // (F * k) - 2) // 4 * ncp))
    for c in sets:
        c["nn"].fill_(n0)
    expand_fn(sets[0])()
    torch.cuda.synchronize()
    assert int(sets[0]["st"].abs().sum()) == 0
    nbytes = B * F * V * 4
    out["expand"] = {"workload": f"batch {B}, {F} frontier rows of {V} logits, k = {k}",
                     "us_per_call": round(us_exp, 3), "bytes": nbytes,
                     "GBps": round(nbytes / (us_exp * 1e-6) / 1e9, 1),
                     "roofline": {"bound": "hbm", "achieved": round(nbytes / (us_exp * 1e-6) / 1e9, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(nbytes / (us_exp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
                     "rows_per_s": B * F / (us_exp * 1e-6)}

    m = MERGE_SHAPE
    toks, lens, root = make_candidates(m["batch"], m["n_cand"], m["max_len"], m["vocab"], seed)
    ct, cl, rt = (torch.from_numpy(x).to(dev) for x in (toks, lens, root))
    outs = [torch.empty((m["batch"], m["n_max"]), dtype=torch.int32, device=dev) for _ in range(2)]
    nn_m = torch.empty(m["batch"], dtype=torch.int32, device=dev)
    no_m = torch.empty(toks.shape, dtype=torch.int32, device=dev)
    st_m = torch.empty(m["batch"], dtype=torch.int32, device=dev)

    def merge_fn():
        tv.tree_merge_candidates(ct, cl, rt, m["n_max"], tokens=outs[0], parent=outs[1], n_nodes=nn_m,
                                 node_of=no_m, status=st_m)

    us_merge = timed([merge_fn], reps)
    assert int(st_m.abs().sum()) == 0
    out["merge"] = {"workload": f"batch {m['batch']}, {m['n_cand']} candidates of up to {m['max_len']} tokens",
                    "us_per_call": round(us_merge, 3), "trees_per_s": m["batch"] / (us_merge * 1e-6),
                    "nodes_per_s": float(nn_m.sum().item()) / (us_merge * 1e-6),
                    "roofline": {"bound": "latency", "note": "one workgroup per request, a few KB each"}}

    q = POOL_SHAPE
    Bp, bs = q["batch"], q["block"]
    mapped = q["prefix"] // bs
    max_blocks = (q["prefix"] + q["nodes"]) // bs + 1
    num_blocks = Bp * max_blocks
    perm = np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)
    table = np.full((Bp, max_blocks), -1, dtype=np.int32)
    table[:, :mapped] = perm[:Bp * mapped].reshape(Bp, mapped)
    free = np.concatenate([perm[Bp * mapped:], np.full(Bp * mapped, -1, dtype=np.int32)])
    d_table = torch.from_numpy(table).to(dev)
    d_nblk = torch.full((Bp,), mapped, dtype=torch.int32, device=dev)
    d_free = torch.from_numpy(free).to(dev)
    d_count = torch.tensor([num_blocks - Bp * mapped], dtype=torch.int32, device=dev)
    d_pre = torch.full((Bp,), q["prefix"], dtype=torch.int32, device=dev)
    d_n = torch.full((Bp,), q["nodes"], dtype=torch.int32, device=dev)
    d_new = torch.full((Bp,), q["prefix"] + q["accepted"], dtype=torch.int32, device=dev)
    d_spec = torch.empty(Bp, dtype=torch.int32, device=dev)
    d_st = torch.empty(Bp, dtype=torch.int32, device=dev)
    d_st2 = torch.empty(Bp, dtype=torch.int32, device=dev)

    def pool_fn():   # allocation then release: the pool returns to the same state
        tv.kv_alloc_tree_blocks(d_table, d_nblk, d_pre, d_n, d_free, d_count, block_size=bs,
                                spec_from=d_spec, status=d_st)
        tv.kv_release_blocks(d_table, d_nblk, d_new, d_free, d_count, block_size=bs, status=d_st2)

    us_pool = timed([pool_fn], reps)
    assert int(d_st.abs().sum()) == 0 and int(d_st2.abs().sum()) == 0
    out["pool"] = {"workload": f"batch {Bp}, {q['nodes']}-node trees after {q['prefix']}-token prefixes, "
                               f"{bs}-token blocks: allocate {(q['prefix'] + q['nodes']) // bs - mapped}, "
                               f"release {(q['prefix'] + q['nodes']) // bs - (q['prefix'] + q['accepted'] + bs - 1) // bs} per request",
                   "us_per_alloc_and_release": round(us_pool, 3),
                   "roofline": {"bound": "latency", "note": "one workgroup, one thread per request"}}

    out["_inputs"] = dict(n0=n0, k=k, n_max=n_max, B=B, F=F, front=front_host, rows=rows_host, toks=toks,
                          lens=lens, root=root, pool=(table, free, mapped, num_blocks))

    # expected acceptance length of a batch of trees (tree-budget calibration)
    from tree_verification_amd.workloads import make_budget_trees
    bt = BUDGET_SHAPE
    bpar, bn, bprob = make_budget_trees(bt["batch"], bt["n_max"], seed)
    d_bpar, d_bn, d_bprob = (torch.from_numpy(x).to(dev) for x in (bpar, bn, bprob))
    d_reach = torch.empty(bpar.shape, dtype=torch.float64, device=dev)
    d_al = torch.empty(bt["batch"], dtype=torch.float64, device=dev)
    d_bst = torch.empty(bt["batch"], dtype=torch.int32, device=dev)

    def budget_fn():
        tv.tree_expected_accept_length(d_bpar, d_bn, d_bprob, reach=d_reach, expected_len=d_al, status=d_bst)

    us_budget = timed([budget_fn], reps)
    assert int(d_bst.abs().sum()) == 0
    out["_budget"] = {"workload": f"batch {bt['batch']} trees of up to {bt['n_max']} nodes "
                                  f"({int(bn.sum())} nodes), per-node acceptance probabilities",
                      "us_per_call": round(us_budget, 3), "trees_per_s": bt["batch"] / (us_budget * 1e-6),
                      "roofline": {"bound": "latency", "note": "one wavefront per tree, ~1.5 KB read each"}}
    if not args.no_cpu_baseline:
        from oracle.budget import expected_length
        t0 = time.perf_counter()
        expected_length(bpar.tolist(), bn.tolist(), bprob.tolist(), bt["n_max"])
        el = time.perf_counter() - t0
        out["_budget"]["cpu_oracle"] = {"us_per_call": el * 1e6, "cores": 1,
                                        "sample": f"all {bt['batch']} trees, {el:.3f} s"}
    return out


# Tree-budget table ([cohere] goodput = AL / ITL, an offline lookup of the best
# draft budget per batch size; [guide] "Dynamic Tree Budget Calibration").
# Candidate trees are expansion schedules (node counts 2, 4, 7, 15, 28, 61);
# every drafted node is accepted with probability BUDGET_ALPHA when tested
# ([chapter]'s representative alpha).  Latencies are measured for this path's
# step at the 8B layer shape (one tree-attention layer, stochastic verification,
# compaction).  A second column prices a whole round with a stated model of the
# parts this path does not build: the target's 32 attention layers as 32 x the
# measured layer, plus its dense weights read once per round or its GEMMs,
# whichever is slower (8.03e9 bf16 parameters, 8 TB/s, 2.5 PFLOP/s).
BUDGET_SCHEDULES = ([1], [1, 1, 1], [2, 1, 1], [2, 2, 1, 1], [3, 2, 1, 1, 1], [4, 2, 2, 1, 1])
BUDGET_BATCHES = (1, 4, 16, 64)
BUDGET_ALPHA = 0.7
BUDGET_LAYER = dict(prefix=2048, n_q_heads=32, n_kv_heads=8, head_dim=128, vocab=128256, block=16, layers=32,
                    params=8.03e9)


def budget_table(args, dev):
    import torch
    from tree_verification_amd import binding as tv
    from tree_verification_amd.workloads import schedule_tree

    L = BUDGET_LAYER
    P, Hq, Hkv, D, V, bs = L["prefix"], L["n_q_heads"], L["n_kv_heads"], L["head_dim"], L["vocab"], L["block"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    shapes = [schedule_tree(sch) for sch in BUDGET_SCHEDULES]
    n_max = max(len(x) for x in shapes)

    # acceptance lengths of the candidate shapes, on the GPU
    par_all = np.full((len(shapes), n_max), -1, dtype=np.int32)
    nn_all = np.array([len(x) for x in shapes], dtype=np.int32)
    prob = np.zeros((len(shapes), n_max))
    for i, x in enumerate(shapes):
        par_all[i, :len(x)] = x
        prob[i, 1:len(x)] = BUDGET_ALPHA
    _, al_d, st_d = tv.tree_expected_accept_length(torch.from_numpy(par_all).to(dev),
                                                   torch.from_numpy(nn_all).to(dev),
                                                   torch.from_numpy(prob).to(dev))
    torch.cuda.synchronize()
    assert int(st_d.abs().sum()) == 0
    al = al_d.cpu().tolist()

    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    a0.record()
    torch.cuda._sleep(20_000_000)
    a1.record()
    torch.cuda.synchronize()
    cyc_per_s = 20_000_000 / (a0.elapsed_time(a1) * 1e-3)

    def timed(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for _ in range(reps):
            fn()
        host_s = time.perf_counter() - h0
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(cyc_per_s * (2.0 * host_s + 2e-3)))   # holds the stream while the calls queue
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    rows = []
    for B in BUDGET_BATCHES:
        row = []
        for si, par in enumerate(shapes):
            N = len(par)
            nblk = (P + N + bs - 1) // bs
            q = torch.randn((B, N, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
            kc = torch.randn((B * nblk, Hkv, bs, D), generator=gen, device=dev).to(torch.bfloat16)
            vc = torch.randn((B * nblk, Hkv, bs, D), generator=gen, device=dev).to(torch.bfloat16)
            table = torch.arange(B * nblk, dtype=torch.int32, device=dev).view(B, nblk)
            pre = torch.full((B,), P, dtype=torch.int32, device=dev)
            nn = torch.full((B,), N, dtype=torch.int32, device=dev)
            pp = torch.from_numpy(np.tile(par, (B, 1))).to(dev)
            tl = torch.randn((B, N, V), generator=gen, device=dev) * 3.0
            dl = tl + torch.randn((B, N, V), generator=gen, device=dev)
            tok = torch.zeros((B, N), dtype=torch.int32, device=dev)
            if N > 1:   # children drawn from the parent's draft row (Gumbel-max)
                pidx = torch.from_numpy(par[1:].astype(np.int64)).to(dev)
                u = torch.rand((B, N - 1, V), generator=gen, device=dev).clamp_min_(1e-30)
                tok[:, 1:] = (dl[:, pidx, :] - torch.log(-torch.log(u))).argmax(-1).to(torch.int32)
                del u
            ua = torch.rand((B, N), generator=gen, device=dev)
            us = torch.rand((B, N), generator=gen, device=dev)
            out = torch.empty_like(q)
            bufs = [torch.empty((B, N), dtype=torch.int32, device=dev) for _ in range(3)]
            ints = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(6)]

            def attn():
                tv.tree_attn_forward(q, kc, vc, table, pre, nn, pp, out=out, status=ints[0])

            def verify():
                tv.tree_verify_stochastic(tl, dl, tok, pp, nn, ua, us, path=bufs[0], path_len=ints[1],
                                          out_tokens=bufs[1], status=ints[2])

            def compact():
                tv.kv_compact_accepted(kc, vc, table, pre, bufs[0], ints[1], src_pos=bufs[2], new_len=ints[3],
                                       status=ints[4])

            attn(), verify(), compact()
            torch.cuda.synchronize()
            assert int(ints[0].abs().sum()) == 0 and int(ints[2].abs().sum()) == 0
            t_attn, t_ver, t_cmp = timed(attn), timed(verify), timed(compact)
            t_step = t_attn + t_ver + t_cmp
            dense = max(L["params"] * 2 / (HBM_PEAK_GBS * 1e9), 2 * L["params"] * B * N / 2.5e15) * 1e6
            t_round = dense + L["layers"] * t_attn + t_ver + t_cmp
            row.append(dict(shape=si, nodes=N, al=al[si], us_attn=t_attn, us_verify=t_ver, us_compact=t_cmp,
                            us_step=t_step, us_round_model=t_round))
            print(json.dumps({"batch": B, "schedule": BUDGET_SCHEDULES[si], **row[-1]}), flush=True)
            del q, kc, vc, tl, dl, out
            torch.cuda.empty_cache()
        rows.append(row)

    best_step = tv.tree_budget_select(al, [[r["us_step"] for r in row] for row in rows])
    best_round = tv.tree_budget_select(al, [[r["us_round_model"] for r in row] for row in rows])
    result = {"table": "tree budget", "alpha": BUDGET_ALPHA, "batches": list(BUDGET_BATCHES),
              "schedules": [list(s) for s in BUDGET_SCHEDULES], "nodes": [len(x) for x in shapes], "al": al,
              "best_shape_step": best_step, "best_shape_round_model": best_round,
              "rows": rows}
    print(json.dumps(result), flush=True)
    if args.budget_out:
        with open(args.budget_out, "w") as f:
            f.write(budget_markdown(result))


def budget_markdown(r) -> str:
    lines = ["| batch | schedule | nodes | AL | attention us | verify us | compact us | step us | "
             "tokens/s (step) | round us (model) | tokens/s (round model) |",
             "|---:|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for bi, B in enumerate(r["batches"]):
        for x in r["rows"][bi]:
            s = x["shape"]
            mark1 = " **best**" if r["best_shape_step"][bi] == s else ""
            mark2 = " **best**" if r["best_shape_round_model"][bi] == s else ""
            lines.append(f"| {B} | {r['schedules'][s]} | {x['nodes']} | {x['al']:.3f} | {x['us_attn']:.1f} | "
                         f"{x['us_verify']:.1f} | {x['us_compact']:.1f} | {x['us_step']:.1f} | "
                         f"{B * x['al'] / (x['us_step'] * 1e-6):,.0f}{mark1} | {x['us_round_model']:.0f} | "
                         f"{B * x['al'] / (x['us_round_model'] * 1e-6):,.0f}{mark2} |")
    return "\n".join(lines) + "\n"


def construction_oracle(out):
    """The oracle's construction functions, timed on the host on (a sample of) the
    same inputs the GPU timings used."""
    from oracle.construct import expand_level, merge_candidates
    x = out["_inputs"]
    n0, k, n_max, B, F = x["n0"], x["k"], x["n_max"], x["B"], x["F"]
    front_host, rows_host, toks, lens, root = x["front"], x["rows"], x["toks"], x["lens"], x["root"]
    m = MERGE_SHAPE
    t0 = time.perf_counter()
    expand_level([0] * n0, [-1] + [0] * (n0 - 1), n0, list(front_host[0]), list(rows_host[0]), k, n_max)
    el = time.perf_counter() - t0
    out["expand"]["cpu_oracle"] = {"us_per_call": el * B * 1e6, "cores": 1,
                                   "sample": f"request 0 of the batch ({F} rows), {el:.2f} s, scaled by {B}"}
    t0 = time.perf_counter()
    for b in range(m["batch"]):
        merge_candidates(int(root[b]), [list(toks[b, i, :lens[b, i]]) for i in range(m["n_cand"])], m["n_max"])
    el = time.perf_counter() - t0
    out["merge"]["cpu_oracle"] = {"us_per_call": el * 1e6, "cores": 1, "sample": f"all {m['batch']} requests, {el:.3f} s"}
    from oracle.pool import alloc_tree_blocks, release_blocks
    q = POOL_SHAPE
    table, free, mapped, num_blocks = x["pool"]
    Bp = q["batch"]
    t0 = time.perf_counter()
    t, nb, f, c, _, _ = alloc_tree_blocks(table, np.full(Bp, mapped), np.full(Bp, q["prefix"]),
                                          np.full(Bp, q["nodes"]), free, num_blocks - Bp * mapped,
                                          block_size=q["block"], num_blocks=num_blocks)
    release_blocks(t, nb, np.full(Bp, q["prefix"] + q["accepted"]), f, c, block_size=q["block"],
                   num_blocks=num_blocks)
    el = time.perf_counter() - t0
    out["pool"]["cpu_oracle"] = {"us_per_call": el * 1e6, "cores": 1, "sample": f"all {Bp} requests, {el:.4f} s"}


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
SIMD_COUNT = 256 * 4      # 256 CUs of four SIMDs
XCD_COUNT = 8             # GRBM_GUI_ACTIVE is reported summed over the XCDs


def mfma_summary(run_dir: str, workload: str):
    """Matrix-core use of the attention kernel from one rocprofv3 --pmc run:
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI-active cycles of one XCD * SIMDs)
    (rocprofv3's MfmaUtil, which takes GRBM_GUI_ACTIVE's maximum over the XCDs;
    the csv holds their sum), and the bf16 MFMA flops executed
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512) beside the algorithmic flops of the same
    call.  The dispatch timestamps give the duration and the implied clock."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            if "tree_attn_kernel" not in name:
                continue
            key = "tree_attn_kernel"
            d = per.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    if "tree_attn_kernel" not in per:
        raise SystemExit(f"no tree_attn_kernel dispatches in {run_dir}")
    from tree_verification_amd.workloads import make_workload
    wl = make_workload(workload, with_logits=False)
    P, n = wl.prefix_len.astype(np.int64), wl.n_nodes.astype(np.int64)
    flops = sum(4 * int(n[b]) * wl.n_q_heads * wl.head_dim * int(P[b]) for b in range(wl.batch))
    for b in range(wl.batch):
        par = wl.parent[b]
        depth = np.zeros(int(n[b]), dtype=np.int64)
        for u in range(1, int(n[b])):
            depth[u] = depth[par[u]] + 1
        flops += int(4 * wl.n_q_heads * wl.head_dim * (depth + 1).sum())
    lines = ["| kernel | dispatches | us | GUI-active cycles per XCD | implied GHz | MFMA busy % | "
             "bf16 MFMA flops executed | algorithmic flops | executed TFLOP/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for key, disp in per.items():
        vals = [d for d in disp.values() if all(c in d for c in MFMA_COUNTERS)]
        if not vals:
            continue
        gui = sum(d["GRBM_GUI_ACTIVE"] for d in vals) / len(vals) / XCD_COUNT
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in vals) / len(vals)
        mops = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in vals) / len(vals) * 512
        us = sum(d["ns"] for d in vals) / len(vals) / 1e3
        alg = f"{flops:,}" if key == "tree_attn_kernel" else "—"
        lines.append(f"| `{key}` | {len(vals)} | {us:.1f} | {gui:,.0f} | {gui / (us * 1e3):.2f} | "
                     f"{100 * busy / (gui * SIMD_COUNT):.1f} | {mops:,.0f} | {alg} | {mops / (us * 1e-6) / 1e12:.1f} |")
    table = "\n".join(lines) + "\n"
    print(table)
    return table


def widen_table(wl, tokens: int):
    """Give every request a block table of ceil(tokens / block) entries (-1 past
    the blocks it owns): a table sized for a longer context than it uses."""
    mb = max(wl.max_blocks, -(-tokens // wl.block_size))
    t = np.full((wl.batch, mb), -1, dtype=np.int32)
    t[:, :wl.max_blocks] = wl.block_table
    wl.block_table = t
    wl.max_blocks = mb
    return wl


def acceptance_stats(args, dev, tv, make_workload):
    """Accepted length per round over several seeds of the workload: the
    histogram of K (accepted drafts; a round emits K + 1 tokens), P(K >= k) and
    the acceptance rate by depth (tests of a child at depth d that accept, over
    all tests at depth d), from stochastic verification on the GPU."""
    import torch
    from tree_verification_amd.workloads import seed_for
    hist, tested, accepted = {}, {}, {}
    ks = []
    seeds = [seed_for(args.config, extra=1 + i) for i in range(max(0, args.accept_seeds))]
    for sd in seeds:
        wl = make_workload(args.config, seed=sd)
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        p, l, _, st = tv.tree_verify_stochastic(f(wl.target_logits), f(wl.draft_logits), f(wl.tokens),
                                                f(wl.parent), f(wl.n_nodes), f(wl.u_accept), f(wl.u_sample))
        torch.cuda.synchronize()
        p, l, st = p.cpu().numpy(), l.cpu().numpy(), st.cpu().numpy()
        for b in range(wl.batch):
            if st[b]:
                continue
            L = int(l[b])
            K = L - 1
            ks.append(K)
            hist[K] = hist.get(K, 0) + 1
            n = int(wl.n_nodes[b])
            par = wl.parent[b, :n]
            for j in range(L):
                u = int(p[b, j])
                if any(int(par[c]) == u for c in range(1, n)):
                    tested[j + 1] = tested.get(j + 1, 0) + 1
                    if j < K:
                        accepted[j + 1] = accepted.get(j + 1, 0) + 1
        del wl
    if not ks:
        return None
    ks = np.asarray(ks)
    kmax = int(ks.max())
    return {"seeds": seeds, "rounds": int(len(ks)),
            "accepted_len_hist": {str(k): hist[k] for k in sorted(hist)},
            "mean_accepted": float(ks.mean()), "mean_tokens_per_round": float(ks.mean() + 1),
            "p_k_at_least": [float((ks >= k).mean()) for k in range(1, kmax + 1)],
            "acceptance_by_depth": {str(d): round(accepted.get(d, 0) / tested[d], 4) for d in sorted(tested)},
            "tests_by_depth": {str(d): tested[d] for d in sorted(tested)}}


def _cpu_request_step(args):
    """One request-step of the oracle (worker process): tree attention for every
    (node, q-head) row, stochastic verification and KV compaction of request b."""
    b, = args
    from threadpoolctl import threadpool_limits

    from oracle.attention import tree_attention
    from oracle.kv import kv_compact
    from oracle.verify import verify_stochastic
    wl = _CPU_WL
    sl = slice(b, b + 1)
    with threadpool_limits(limits=1):
        tree_attention(wl.q[sl], wl.k_cache, wl.v_cache, wl.block_table[sl], wl.prefix_len[sl], wl.n_nodes[sl],
                       wl.parent[sl], n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                       block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max, sm_scale=wl.sm_scale)
        paths, _, _, _ = verify_stochastic(wl.target_logits[sl], wl.draft_logits[sl], wl.tokens[sl],
                                           wl.parent[sl], wl.n_nodes[sl], wl.u_accept[sl], wl.u_sample[sl],
                                           wl.n_max)
        pth = np.full((1, wl.n_max), -1, dtype=np.int32)
        pth[0, :len(paths[0])] = paths[0]
        kv_compact(wl.k_cache, wl.v_cache, wl.block_table[sl], wl.prefix_len[sl], pth, np.array([len(paths[0])]),
                   block_size=wl.block_size, num_blocks=wl.num_blocks, n_max=wl.n_max)
    return int(wl.n_nodes[b])


_CPU_WL = None


def cpu_info():
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    model = fields.get("model name", "unknown")
    return f"{model} (family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}, " \
           f"stepping {fields.get('stepping', '?')})"


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        import numpy  # noqa: F401  (loads its BLAS)
        libs = [f"{d.get('internal_api')} {d.get('version')}" for d in threadpool_info() if d.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:
        return "unknown"


def cpu_baseline(wl, seconds: float):
    """The oracle, unmodified, on the host's cores: a process pool (one worker per
    core of os.sched_getaffinity, at most 16, each with one BLAS thread) runs
    request-steps of the workload (attention for every node and q-head,
    stochastic verification, compaction) for about `seconds`; requests cycle
    through the batch.  Must run before the GPU is initialised (fork)."""
    import multiprocessing as mp
    global _CPU_WL
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    _CPU_WL = wl
    ctx = mp.get_context("fork")
    done_nodes = 0
    steps = 0
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pending = []
        b = 0
        while True:
            while len(pending) < 2 * cores and (time.perf_counter() - t0 < seconds or steps + len(pending) < cores):
                pending.append(pool.apply_async(_cpu_request_step, ((b,),)))
                b = (b + 1) % wl.batch
            if not pending:
                break
            r = pending.pop(0)
            done_nodes += r.get()
            steps += 1
            if time.perf_counter() - t0 >= seconds and steps >= cores:
                for r in pending:
                    done_nodes += r.get()
                    steps += 1
                break
    el = time.perf_counter() - t0
    _CPU_WL = None
    return {"value": done_nodes / el, "unit": "nodes/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} request-steps of this workload (attention for every node and q-head, "
                      f"stochastic verification, KV compaction) on a pool of {cores} worker processes, "
                      f"{el:.1f} s, one BLAS thread each",
            "cpu_model": cpu_info(), "blas": blas_info()}


if __name__ == "__main__":
    main()
