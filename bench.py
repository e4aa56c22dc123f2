#!/usr/bin/env python3
"""Benchmark of the fused LM-head projection + exact top-k on one MI355X.

Default workload: binary head V=248,320, H=5,120, k=50, M=1, no bias, group
128 -- the head of the lm-head-topk page's measurement (its intro and section
"Measured"), with seeded synthetic weights (no trained checkpoint is used).

One step = one library call on inputs already resident in HBM; at this shape
it is one kernel launch (chunk scoring, per-chunk selection, and the final
merge in the launch's last workgroup).  The packed head is
198.7 MB, smaller than the 256 MB Infinity Cache, so the timed loop rotates
--copies bitwise-identical packed copies (4 x 198.7 MB) to make the weights
come from HBM; a single-copy (cache-served) figure is reported beside it.
--sample adds the token draw of the logits-processor page's usage example
(temperature 0.7, top_k 50, top_p 0.9) to every call.

Order: inputs; the auxiliary measurements (graph replay, cache-served single
copy, the box's plain read and copy rates), which also bring an idle GPU to
its steady clocks; the --warmup untimed steps; the --steps timed steps; the
scoring kernel's own duration (events on its dispatch); the materialized
comparison; the CPU oracle.

Printed: one JSON line (see the end of main()).  Kernel times come from HIP
events recorded on the stream the kernels run on; `roofline.traffic` comes from
rocprofv3 counter runs summarised under profiles/ (see --summarize-pmc).

Profiling helpers (CPU only, no GPU work):
  --summarize-trace DIR   turn a `rocprofv3 --kernel-trace --stats -d DIR` run of
                          this script into profiles/<name>_kernel_trace.txt
  --summarize-pmc F W     turn two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
                          runs into profiles/<name>_traffic.{txt,json}
"""

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/token + achieved HBM GB/s, binary head V=248,320 H=5,120 k=50, M=1"
HBM_PEAK_GBPS = 8000.0
SCORE_KERNEL = "k_binary_chunk"
COPY_BYTES = 1 << 30
KERNEL_SOURCES = ["lm_head_projection_amd/csrc/lmtopk_binary.hip",
                  "lm_head_projection_amd/csrc/lmtopk_chunk.hpp",
                  "lm_head_projection_amd/csrc/lmtopk_device.hpp",
                  "lm_head_projection_amd/csrc/lmtopk_sample.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    # an MI355X left idle (input set-up, a sleep) runs the first ~2,000 calls
    # about 10 % slower; the untimed warm-up brings it to its steady state
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--copies", type=int, default=4, help="rotated packed heads (defeats the 256 MB MALL)")
    p.add_argument("--M", type=int, default=1)
    p.add_argument("--k", type=int, default=50)
    p.add_argument("--V", type=int, default=248320)
    p.add_argument("--H", type=int, default=5120)
    p.add_argument("--bias", action="store_true")
    p.add_argument("--chunk-rows", type=int, default=0)
    p.add_argument("--lse", action="store_true", help="also return each row's log-sum-exp")
    p.add_argument("--sample", action="store_true",
                   help="also draw one token per row (temperature 0.7, top_k 50, top_p 0.9)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-reps", type=int, default=5, help="oracle calls timed for cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-compare", action="store_true", help="skip the materialized-logits comparison")
    p.add_argument("--name", default="binary_v248320_h5120_k50_m1",
                   help="summary name for the --summarize-* commands")
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    p.add_argument("--summarize-counters", metavar="DIR",
                   help="turn a `rocprofv3 --pmc <SQ counters> GRBM_GUI_ACTIVE` run into "
                        "profiles/<name>_counters.txt")
    p.add_argument("--no-aux", action="store_true",
                   help="skip the graph replay and single-copy measurements (for profiled runs: "
                        "every scoring dispatch then reads rotated copies)")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    return p.parse_args()


# ---------------------------------------------------------------------------
# HIP events through the HIP runtime instance torch has loaded
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("libamdhip64 is not loaded")
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)


# ---------------------------------------------------------------------------
# rocprofv3 summaries (host-side parsing only)
# ---------------------------------------------------------------------------
def _csv_rows(pattern_dir, suffix):
    files = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return files, rows


def summarize_trace(d, name, command):
    files, rows = _csv_rows(d, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    out = os.path.join(ROOT, "profiles", f"{name}_kernel_trace.txt")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write(f"rocprofv3 kernel trace summary: {name}\n")
        f.write(f"command: {command}\n")
        f.write(f"kernel sources sha256[:16]: {kernel_source_hash()}\n\n")
        f.write(f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel\n")
        for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
            nm = r.get("Name", r.get("KernelName", "?"))
            f.write(f"{int(r['Calls']):>7} {float(r['AverageNs'])/1e3:>10.2f} "
                    f"{float(r['MinNs'])/1e3:>10.2f} {float(r['MaxNs'])/1e3:>10.2f} "
                    f"{float(r.get('Percentage', 0)):>8.2f}  {nm[:150]}\n")
    print(f"wrote {out}")


def _pmc_per_dispatch(d, counter):
    files, rows = _csv_rows(d, "counter_collection.csv")
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        nm = r.get("Kernel_Name", "")
        per.setdefault(nm, []).append(float(r["Counter_Value"]))
    return per


def summarize_pmc(fetch_dir, write_dir, name, command):
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")

    def pick(per, sub):
        ks = [k for k in per if sub in k]
        if not ks:
            raise SystemExit(f"no kernel matching {sub!r}: {list(per)[:8]}")
        vals = [v for k in ks for v in per[k]]
        return statistics.median(vals), len(vals)

    copy_sub = "MulFunctor"  # the plain copy of plain_copy_gbps
    f_copy, _ = pick(fetch, copy_sub)
    w_copy, _ = pick(write, copy_sub)
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    f_k, nf = pick(fetch, SCORE_KERNEL)
    w_k, nw = pick(write, SCORE_KERNEL)
    fetch_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    res = {"kernel": SCORE_KERNEL, "kernel_source_sha256_16": kernel_source_hash(),
           "fetch_kib_per_dispatch": f_k, "write_kib_per_dispatch": w_k,
           "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "traffic_bytes_per_launch": fetch_b + write_b, "dispatches": [nf, nw],
           "command": command}
    base = os.path.join(ROOT, "profiles", f"{name}_traffic")
    with open(base + ".json", "w") as f:
        json.dump(res, f, indent=1)
    with open(base + ".txt", "w") as f:
        f.write(f"rocprofv3 HBM traffic of {SCORE_KERNEL}: {name}\n")
        f.write(f"command: {command}\n")
        f.write(f"calibration: plain copy of {COPY_BYTES} B read + {COPY_BYTES} B written "
                f"reads FETCH_SIZE {f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB -> scale "
                f"{f_scale:.4f} / {w_scale:.4f}\n")
        f.write(f"{SCORE_KERNEL}: FETCH_SIZE {f_k:.0f} KiB/dispatch -> {fetch_b/1e6:.3f} MB; "
                f"WRITE_SIZE {w_k:.0f} KiB/dispatch -> {write_b/1e6:.3f} MB "
                f"(median of {nf} / {nw} dispatches)\n")
    print(f"wrote {base}.json/.txt")


def summarize_counters(d, name, command):
    """Per-dispatch medians of the SQ / GRBM counters of every kernel, and for
    the scoring kernel the derived figures rocprof itself defines: VALU busy =
    100 * sum(SQ_ACTIVE_INST_VALU) / CU_NUM / max(GRBM_GUI_ACTIVE), mean
    occupancy = 400 * sum(SQ_WAVE_CYCLES) / max(GRBM_GUI_ACTIVE) / CU_NUM / 32
    (percent of 32 waves per CU); CU_NUM = 256.  The per-dispatch
    GRBM_GUI_ACTIVE of the CSV is the sum over the 8 XCDs, so its maximum
    over them is taken as that sum / 8 (the XCDs run the dispatch together)."""
    files, rows = _csv_rows(d, "counter_collection.csv")
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for r in rows:
        per.setdefault(r.get("Kernel_Name", "?"), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    out = os.path.join(ROOT, "profiles", f"{name}_counters.txt")
    cu = 256
    with open(out, "w") as f:
        f.write(f"rocprofv3 counters: {name}\n")
        f.write(f"command: {command}\n")
        f.write(f"kernel sources sha256[:16]: {kernel_source_hash()}\n\n")
        for kern, cs in sorted(per.items(), key=lambda kv: SCORE_KERNEL not in kv[0]):
            med = {c: statistics.median(v) for c, v in cs.items()}
            n = max(len(v) for v in cs.values())
            f.write(f"{kern[:120]}  ({n} dispatches, medians)\n")
            for c in sorted(med):
                f.write(f"  {c:24s} {med[c]:.6g}\n")
            gui = med.get("GRBM_GUI_ACTIVE")
            if gui:
                gui /= 8.0  # one XCD's busy cycles
                f.write(f"  busy cycles per XCD      {gui:.6g} ({gui / 2.4e3:.1f} us at 2.4 GHz)\n")
                if "SQ_ACTIVE_INST_VALU" in med:
                    f.write(f"  VALU busy                {100 * med['SQ_ACTIVE_INST_VALU'] / cu / gui:.1f} %\n")
                if "SQ_WAVE_CYCLES" in med:
                    f.write(f"  mean occupancy           {400 * med['SQ_WAVE_CYCLES'] / gui / cu / 32:.1f} % "
                            f"of 32 waves per CU\n")
            if med.get("SQ_WAVES") and "SQ_INSTS_VALU" in med:
                f.write(f"  VALU instructions / wave {med['SQ_INSTS_VALU'] / med['SQ_WAVES']:.0f}\n")
            f.write("\n")
    print(f"wrote {out}")


def load_traffic(name):
    fn = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    return t["traffic_bytes_per_launch"]


# ---------------------------------------------------------------------------
# the benchmark
# ---------------------------------------------------------------------------
def algorithmic_score_bytes(M, V, H, k, bias, chunk_rows, lt):
    """Packed head + bias + activations and scales read, plus the chunks'
    candidate lists written (k entries of 8 bytes per row and chunk, with the
    chunk count the library plans for these sizes)."""
    wq_b, ws_b = lt.packed_bytes(V, H)
    C, n_chunks, _ = lt.binary_plan(M, V, H, k, chunk_rows)
    kc = min(k, C)
    return wq_b + ws_b + (4 * V if bias else 0) + M * H + 4 * M + M * n_chunks * kc * 8


def workload_name(args):
    """Name of this workload's profile summaries (profiles/<name>_*)."""
    n = f"binary_v{args.V}_h{args.H}_k{args.k}_m{args.M}"
    n += "_bias" if args.bias else ""
    n += "_lse" if args.lse else ""
    n += "_sample" if args.sample else ""
    n += f"_c{args.chunk_rows}" if args.chunk_rows else ""
    return n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(args, W, act_q, act_scale, bias):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    V, H, M = args.V, args.H, args.M
    signs = np.empty((V, H), dtype=np.int8)
    scales = np.empty((V, H // 128), dtype=np.float32)
    for v0 in range(0, V, 8192):  # logical packing: offline preparation, not timed
        signs[v0:v0 + 8192], scales[v0:v0 + 8192] = oracle.pack_logical(W[v0:v0 + 8192])
    times = []
    for _ in range(args.cpu_reps):
        t = time.perf_counter()
        L = oracle.project_binary(act_q, act_scale, signs, scales, bias)
        oracle.topk_stable_rows(L, args.k)
        times.append(time.perf_counter() - t)
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    per_call = statistics.median(times)
    return {"value": per_call * 1e6 / M, "unit": "µs/token", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{args.cpu_reps} full oracle calls (fp64 dequantized projection of all "
                      f"{V} rows + stable top-{args.k}) at M={M}; median {per_call:.2f} s per call; "
                      f"BLAS threads {threads}, NumPy elementwise single-threaded; host has "
                      f"{len(os.sched_getaffinity(0))} cores ({cpu_model()})"}


def time_calls(hip, stream, call, n, per_step_events):
    """Run n calls back to back and time them with events on the stream.

    The host enqueues a call in about 14 us, well under the GPU's time per
    call, so after the first call the GPU never waits for the host.  (An
    idle spin kernel in front, to queue every call before the GPU starts,
    made the same calls about 5 us slower each on MI355X.)

    With per_step_events the scoring kernel of every call records its own
    start and end (events attached to its dispatch) and an event after the
    call closes the merge.  Returns (total_ms, [score_ms], [merge_ms])."""
    import torch
    torch.cuda.synchronize()
    ev0, ev1 = hip.event(), hip.event()
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(n)] if per_step_events else None
    hip.record(ev0, stream)
    for i in range(n):
        if evs:
            call(i, (evs[i][0], evs[i][1]))
            hip.record(evs[i][2], stream)
        else:
            call(i, None)
    hip.record(ev1, stream)
    torch.cuda.synchronize()
    total = hip.ms(ev0, ev1)
    score, merge = [], []
    if evs:
        for a, b, c in evs:
            score.append(hip.ms(a, b))
            merge.append(hip.ms(b, c))
    return total, score, merge


def main():
    args = parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.name, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.name, args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.name, args.command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lm_head_projection_amd as lt
    import synthetic

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    M, V, H, k = args.M, args.V, args.H, args.k
    log = lambda s: print(f"[bench] {s}", file=sys.stderr, flush=True)

    # ---- inputs (seeded, synthetic), resident in HBM before timing ----
    t0 = time.time()
    W = synthetic.dense_head(V, H, args.seed)
    x = synthetic.hidden_rows(M, H, args.seed)
    act_q, act_scale = synthetic.quantize_rows_int8(x)
    bias = synthetic.bias_vector(V, args.seed) if args.bias else None
    Wd = torch.from_numpy(W).to(dev)
    wq0, ws0 = lt.pack_binary(Wd)
    del Wd
    copies = [(wq0, ws0)] + [(wq0.clone(), ws0.clone()) for _ in range(args.copies - 1)]
    d_aq = torch.from_numpy(act_q).to(dev)
    d_as = torch.from_numpy(act_scale).to(dev)
    d_b = torch.from_numpy(bias).to(dev) if bias is not None else None
    vals = torch.empty((M, k), dtype=torch.float32, device=dev)
    idx = torch.empty((M, k), dtype=torch.int64, device=dev)
    work = lt.new_workspace(M, V, k, args.chunk_rows, device=dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if args.lse else None
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s (packed head {lt.packed_bytes(V, H)} B x {args.copies})")

    hip = Hip()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    tokens = torch.empty(M, dtype=torch.int64, device=dev) if args.sample else None

    def call(i, ev, rot=args.copies):
        wq, ws = copies[i % rot]
        smp = lt.Sampling(0.7, min(50, k), 0.9, 0.0, seed=args.seed, offset=i) if args.sample else None
        lt.lm_head_topk_binary(d_aq, d_as, wq, ws, bias=d_b, k=k, vocab_size=V,
                               chunk_rows=args.chunk_rows, out=(vals, idx), workspace=work,
                               score_events=ev, lse=lse, sampling=smp, tokens=tokens)

    # auxiliary measurements first: the plain read and copy of 1 GiB (which
    # sweep the caches and the TLB), then the calls' own auxiliary runs, and
    # before the warm-up a run of the timed calls themselves, so that the
    # timed steps start from the state the calls keep in steady decoding
    # (an idle GPU reaches its steady clocks, and the caches and TLB hold
    # what the calls use, not what the 1 GiB probes left)
    aux_calls = max(args.steps, 1000)
    read_gbps = plain_read_gbps(hip, stream, dev)
    stream_gbps = plain_copy_gbps(hip, stream, dev)
    graph_us = warm_us = None
    if not args.no_aux:
        graph_us = graph_replay_us(args, call, hip, stream, vals, idx)
        # one packed copy only: served from the 256 MB Infinity Cache
        warm_ms, _, _ = time_calls(hip, stream, lambda i, ev: call(i, ev, 1), aux_calls, False)
        warm_us = warm_ms / aux_calls * 1e3
    log(f"hipGraph replay {graph_us} us/step; single-copy (cache) {warm_us} us/step; "
        f"plain 1 GiB read {read_gbps:.0f} GB/s, copy {stream_gbps:.0f} GB/s (read + written)")
    time_calls(hip, stream, call, aux_calls, False)

    for i in range(args.warmup):
        call(i, None)
    torch.cuda.synchronize()

    # timed region: K steps, synchronised on both sides
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    total_ms, _, _ = time_calls(hip, stream, call, args.steps, per_step_events=False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (GPU events); wall {wall * 1e3:.1f} ms")

    # the scoring kernel's own duration: events attached to its dispatch, on
    # the stream it runs on (same rotation, right after the timed steps)
    _, score_ms, merge_ms = time_calls(hip, stream, call, aux_calls, per_step_events=True)
    score_us = statistics.mean(score_ms) * 1e3
    merge_us = statistics.mean(merge_ms) * 1e3
    log(f"scoring kernel {score_us:.2f} us, then {merge_us:.2f} us to the call's closing event")
    # per-call spread: scoring kernel start to the call's closing event
    call_us = sorted((a + b) * 1e3 for a, b in zip(score_ms, merge_ms))
    pct = lambda q: round(call_us[min(len(call_us) - 1, int(q * len(call_us)))], 3)
    log(f"per call p10/p50/p90 {pct(0.1)}/{pct(0.5)}/{pct(0.9)} us")

    # (plain_copy_gbps above also serves as the counter calibration of
    # --summarize-pmc: a copy of known size)

    head_bytes = sum(lt.packed_bytes(V, H))
    alg_bytes = algorithmic_score_bytes(M, V, H, k, args.bias, args.chunk_rows, lt)
    achieved = alg_bytes / (score_us * 1e-6) / 1e9
    traffic = load_traffic(workload_name(args))  # null unless counters of this workload exist
    plan_c, plan_n, plan_w = lt.binary_plan(M, V, H, k, args.chunk_rows)

    result = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3 / M, 3),
        "unit": "µs/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x 1-bit integer dots, fp32 accumulate",
        "data": "synthetic (seeded N(0,1)/sqrt(H) head and hidden rows; int8 symmetric activations)",
        "config": {"workload": f"binary head V={V} H={H} k={k} M={M} group 128"
                               f"{' +bias' if args.bias else ''}{' +lse' if args.lse else ''}"
                               f"{' +sample(T 0.7, top_k 50, top_p 0.9)' if args.sample else ''}, "
                               f"{args.copies} rotated packed copies",
                   "V": V, "H": H, "k": k, "M": M, "bias": bool(args.bias), "lse": bool(args.lse),
                   "sample": bool(args.sample),
                   "chunk_rows": plan_c, "chunks": plan_n, "waves_per_chunk": plan_w,
                   "rotated_copies": args.copies},
        "gbps": round(head_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "head_bytes": head_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": SCORE_KERNEL, "algorithmic_bytes": alg_bytes,
                     "avg_kernel_us": round(score_us, 3)},
        "kernels_us": {"score_select_merge": round(score_us, 3),
                       "kernel_end_to_call_event": round(merge_us, 3)},
        "per_call_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "graph_replay_us_per_step": graph_us,
        "plain_read_gbps_1gib": round(read_gbps, 1),
        "plain_copy_gbps_1gib": round(stream_gbps, 1),
        "cache_served_single_copy": None if warm_us is None else {
            "us_per_token": round(warm_us / M, 3),
            "gbps": round(head_bytes / (warm_us * 1e-6) / 1e9, 1)},
    }

    if not args.no_compare:
        result["comparison"] = materialized_comparison(args, lt, hip, stream, dev)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(args, W, act_q, act_scale, bias)
    print(json.dumps(result), flush=True)


def graph_replay_us(args, call, hip, stream, vals, idx):
    """The same rotated calls captured once in a hipGraph and replayed (no
    host launch cost per call).  Checks that a replay leaves the eager
    result."""
    import torch
    call(0, None)
    torch.cuda.synchronize()
    ref_v, ref_i = vals.clone(), idx.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(args.copies):
                call(i, None)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    reps = max(1, args.steps // args.copies)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    if not (torch.equal(idx, ref_i) and torch.equal(vals.view(torch.int32), ref_v.view(torch.int32))):
        raise RuntimeError("graph replay result differs from the eager call")
    t, _, _ = time_calls(hip, torch.cuda.current_stream().cuda_stream, lambda i, ev: g.replay(), reps,
                         False)
    del g
    return round(t / (reps * args.copies) * 1e3, 3)


def plain_read_gbps(hip, stream, dev):
    """Achievable HBM read rate on this machine: a plain non-temporal streaming
    read of 1 GiB (lm_head_projection_amd/csrc/probe_read.hip), 256
    workgroups of 1,024 threads, best of 3 runs of 10 launches."""
    import torch
    path = os.path.join(ROOT, "lm_head_projection_amd", "_lib", "libprobe_read.so")
    lib = ctypes.CDLL(path)
    lib.probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_void_p]
    buf = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(256 * 4, dtype=torch.int32, device=dev)
    run = lambda i, ev: lib.probe_read(buf.data_ptr(), COPY_BYTES, sink.data_ptr(), 256, stream)
    for i in range(3):
        if run(i, None) != 0:
            raise RuntimeError("probe_read launch failed")
    best = min(time_calls(hip, stream, run, 10, False)[0] for _ in range(3))
    del buf, sink
    return COPY_BYTES / (best / 10 * 1e-3) / 1e9


def plain_copy_gbps(hip, stream, dev):
    """Achievable HBM rate on this machine for plain streaming: torch's elementwise
    copy of 1 GiB (bytes read + bytes written per second)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    t, _, _ = time_calls(hip, stream, lambda i, ev: torch.mul(src, 1.0, out=dst), 10, False)
    del src, dst
    return 2 * COPY_BYTES / (t / 10 * 1e-3) / 1e9


def materialized_comparison(args, lt, hip, stream, dev):
    """bf16 head + materialized logits + separate top-k, on the same GPU."""
    import torch
    M, V, H, k = args.M, args.V, args.H, args.k
    g = torch.Generator(device=dev).manual_seed(args.seed)
    Wb = (torch.randn((V, H), generator=g, device=dev, dtype=torch.float32) / math.sqrt(H)).to(torch.bfloat16)
    hb = (torch.randn((M, H), generator=g, device=dev, dtype=torch.float32) / math.sqrt(H)).to(torch.bfloat16)
    n = 20
    out = {}

    def mat(i, ev):
        logits = torch.matmul(hb, Wb.t())
        torch.topk(logits.float(), k)

    def dense(i, ev):
        lt.lm_head_topk_dense(hb, Wb, k=k)

    for name, fn in (("torch_bf16_matmul_plus_topk", mat), ("lmtopk_dense_bf16", dense)):
        for i in range(3):
            fn(i, None)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        t, _, _ = time_calls(hip, stream, fn, n, False)
        peak = torch.cuda.max_memory_allocated() - base
        out[name] = {"us_per_call": round(t / n * 1e3, 2),
                     "extra_peak_mib": round(peak / 2**20, 2)}
    logits = torch.matmul(hb, Wb.t()).float()
    for i in range(3):
        lt.topk_logits(logits, k)
    t, _, _ = time_calls(hip, stream, lambda i, ev: lt.topk_logits(logits, k), n, False)
    out["lmtopk_select_on_materialized_fp32"] = {"us_per_call": round(t / n * 1e3, 2)}
    t, _, _ = time_calls(hip, stream, lambda i, ev: torch.topk(logits, k), n, False)
    out["torch_topk_on_materialized_fp32"] = {"us_per_call": round(t / n * 1e3, 2)}
    out["bf16_head_bytes"] = V * H * 2
    del Wb
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
