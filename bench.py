"""Benchmark: fused sampling at B=256, V=2^18 (bf16 logits, grammar bitmask,
penalties, logit bias, mixed per-request settings) on one MI355X.

One step = one full pass of the hot path over the batch: Stage 1 (per-tile
prelude + top-128) and Stage 2 (merge, temperature, top-p / min-p,
Gumbel-max) for all 256 rows, replayed from a hipGraph with the Philox
offset advanced on the device.  Inputs are resident in HBM; sixteen copies
of the logits and bitmask are rotated so the 256 MB last-level cache cannot
serve a step from the previous one.  Exactly --steps steps are timed (wall
clock, synchronised on both sides) for `value`: one graph holds them all
(step i on copy i mod 16) and is replayed once, so the sampler's kernels
run back to back as inside a decode loop's graph.  The median per step
over --median-replays event-timed replays of a sixteen-step graph is
reported beside it.

Printed: one JSON line with the headline rate (sampled tokens/s), the
Stage-1 roofline (algorithmic bytes / mean time of the step's own Stage-1
launch, HIP events, against the 8 TB/s HBM peak), the end-to-end logits
GB/s, the verification latency of the B=64, gamma=4, V=2^17 workload, the
stress legs and other workloads, and the CPU oracle timed on a bounded
sample of the same rows.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
B_HEAD, V_HEAD = 256, 262144
PRIOR, NBIAS = 64, 16


def alg_bytes_per_row(V, prior, nbias, grammar=True, dtype_bytes=2):
    """Bytes one row must move: logits, grammar bitmask, prior list (id +
    count), bias list (id + value), the 32-byte request record and the
    4-byte token."""
    return V * dtype_bytes + ((V + 31) // 32) * 4 * grammar + prior * 8 + nbias * 8 + 32 + 4


def stage1_bytes_per_row(V, prior, nbias, grammar=True, dtype_bytes=2):
    return alg_bytes_per_row(V, prior, nbias, grammar, dtype_bytes) - 4


PROFILE_MD = os.path.join(ROOT, "profiles", "stage1_bf16_c2.md")
# the runs behind profiles/ (from the repository root, TMPDIR=/tmp); the
# summary is written by `python3 bench.py --summarize-rocprof rocprof_out`
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/trace -o run -- "
             "python3 bench.py --steps 40 --warmup 8 --no-cpu --legs c2",
    "FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/FETCH_SIZE -o run -- "
                  "python3 bench.py --steps 8 --warmup 2 --no-cpu --legs c2 --copy-calibration",
    "WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/WRITE_SIZE -o run -- "
                  "python3 bench.py --steps 8 --warmup 2 --no-cpu --legs c2 --copy-calibration",
    "extra": "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/extra -o run -- "
             "python3 bench.py --steps 8 --warmup 2 --no-cpu --median-replays 5 --legs verify,stress,c0,c1,c4",
    "lmhead": "rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/lmhead -o run -- "
              "python3 bench.py --steps 8 --warmup 2 --no-cpu --median-replays 5 --legs lmhead",
}


# the sources the sampling step's Stage-1 launch is built from (its kernel,
# the listed-token waves it runs, the helpers both use, the request layout)
STAGE1_SOURCES = ("ss_device.h", "ss_wavesort.h", "ss_stage1.h", "ss_kernels.h", "ss_stage2.h")


def kernel_source_hash() -> str:
    """sha256 over the Stage-1 sources and the C header: recorded HBM
    counters apply only to the kernel they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_stage1_amd", "csrc")
    files = [os.path.join(csrc, f) for f in STAGE1_SOURCES] + [os.path.join(ROOT, "include", "ss.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per Stage-1 launch from the committed counter summary, or
    None when the kernels changed since it was taken."""
    try:
        with open(PROFILE_MD) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:") or line.startswith("source_sha256:"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def summarize_rocprof(d: str, out: str) -> None:
    """Writes the short summaries kept under profiles/ from the rocprofv3
    runs of PROFILE_CMDS (output directory d)."""
    import csv
    import statistics

    def rows(path):
        with open(path) as fh:
            return list(csv.DictReader(fh))

    def per_shape(trace_csv):
        per = {}
        for r in rows(trace_csv):
            if "ssd::" not in r["Kernel_Name"]:
                continue
            k = (r["Kernel_Name"], int(r["Grid_Size_X"]))
            per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        return per

    def shape_table(per, pick):
        ll = ["| kernel | grid (threads) | calls | avg us | median us |", "|---|---|---|---|---|"]
        for (name, grid), v in sorted(per.items()):
            if pick(name, grid):
                ll.append(f"| {name} | {grid} | {len(v)} | {sum(v) / len(v):.2f} | {statistics.median(v):.2f} |")
        return ll

    B, V = B_HEAD, V_HEAD
    # the sampling step's Stage-1 launch: ceil(B/4) listed-token workgroups
    # plus one workgroup per (row, tile), 256 threads each
    step_grid = ((B + 3) // 4 + B * ((V + 32767) // 32768)) * 256
    per = per_shape(os.path.join(d, "trace", "run_kernel_trace.csv"))
    lines = ["# Stage 1 (bf16), c2 workload: B=256, V=262144, rotating input copies", ""]
    lines += ["Commands (run from the repository root with TMPDIR=/tmp):", ""]
    lines += ["    " + PROFILE_CMDS[k] for k in ("trace", "FETCH_SIZE", "WRITE_SIZE")] + [""]
    lines += ["## rocprofv3 --kernel-trace --stats (kernel_stats.csv, ssd kernels)", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows(os.path.join(d, "trace", "run_kernel_stats.csv")):
        if "ssd::" in r["Name"]:
            lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## per launch shape (kernel_trace.csv)", ""] + shape_table(per, lambda n, g: True)
    s1 = per.get(("void ssd::stage1_kernel<1>(ssd::Stage1Params)", step_grid), [])

    def counter(name):
        rr = rows(os.path.join(d, name, "run_counter_collection.csv"))
        st = [float(r["Counter_Value"]) for r in rr
              if "stage1_kernel<1>" in r["Kernel_Name"] and int(r["Grid_Size"]) == step_grid]
        rd = [float(r["Counter_Value"]) for r in rr if "stream_read_kernel" in r["Kernel_Name"]]
        cp = [float(r["Counter_Value"]) for r in rr if "neg_kernel" in r["Kernel_Name"]]
        avg = lambda v: sum(v) / len(v) if v else float("nan")
        return avg(st), avg(rd), avg(cp)

    f_s1, f_rd, _ = counter("FETCH_SIZE")
    w_s1, _, w_cp = counter("WRITE_SIZE")
    ff = (1 << 30) / 1024.0 / f_rd     # the streaming read fetches 1 GiB with the logits' nt policy
    fw = (128 << 20) / 1024.0 / w_cp   # the copy writes 128 MiB
    traffic = (f_s1 * ff + w_s1 * fw) * 1024.0
    alg = stage1_bytes_per_row(V, PRIOR, NBIAS) * B
    avg_us = sum(s1) / len(s1) if s1 else float("nan")
    lines += ["", "## HBM bytes (rocprofv3 --pmc, KiB per dispatch)", "",
              f"- FETCH_SIZE calibration: ss_stream_read over 1 GiB (16-byte nt loads): {f_rd:.1f} KiB "
              f"-> scale {ff:.4f}",
              f"- WRITE_SIZE calibration: torch.neg writing 128 MiB: {w_cp:.1f} KiB -> scale {fw:.4f}",
              f"- stage1_kernel<bf16>, grid {step_grid} (the step's launch): FETCH_SIZE {f_s1:.1f}, "
              f"WRITE_SIZE {w_s1:.1f}",
              f"- scaled: {f_s1 * ff / 1024:.2f} MiB read, {w_s1 * fw / 1024:.2f} MiB written per launch; "
              f"algorithmic {alg / 2**20:.2f} MiB (ratio {traffic / alg:.3f})",
              f"- Stage-1 average over {len(s1)} launches of that shape: {avg_us:.2f} us -> "
              f"{alg / (avg_us * 1e-6) / 1e9:.1f} GB/s = {alg / (avg_us * 1e-6) / 1e9 / HBM_PEAK_GBPS:.4f} "
              f"of {HBM_PEAK_GBPS:.0f} GB/s", "",
              f"traffic_bytes_per_launch: {int(round(traffic))}",
              f"source_sha256: {kernel_source_hash()}", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))

    # the other workloads, from the "extra" trace
    xd = os.path.join(d, "extra")
    if not os.path.isdir(xd):
        return
    stats = rows(os.path.join(xd, "run_kernel_stats.csv"))
    perx = per_shape(os.path.join(xd, "run_kernel_trace.csv"))
    ll = ["# The other workloads: c3 verification (bounded, per-request draft counts, dense), Stage 1 off "
          "its usual path at c2's shape (log-probability rows, 0.1 %-allowed grammar, more than 128 listed "
          "tokens in one tile), c0, c1, and c4 top-k (512 x 262144 fp32, peaked and flat)", "",
          "Command (run from the repository root with TMPDIR=/tmp):", "", "    " + PROFILE_CMDS["extra"], "",
          "## rocprofv3 --kernel-trace --stats (kernel_stats.csv)", "",
          "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "ssd::" in r["Name"]:
            ll.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                      f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    ll += ["", "## per launch shape (kernel_trace.csv)", ""] + shape_table(perx, lambda n, g: True)
    with open(os.path.join(os.path.dirname(out), "other_workloads.md"), "w") as fh:
        fh.write("\n".join(ll) + "\n")

    # the LM head fused with sampling
    ld = os.path.join(d, "lmhead")
    if not os.path.isdir(ld):
        return
    perl = per_shape(os.path.join(ld, "run_kernel_trace.csv"))
    ll = ["# LM head fused with sampling: B=64, D=4096, V=131072 and B=256, D=4096, V=262144 "
          "(bf16 hidden and weights, synthetic)", "",
          "Command (run from the repository root with TMPDIR=/tmp):", "", "    " + PROFILE_CMDS["lmhead"], "",
          "Grid sizes are in threads (256 per workgroup, 512 with the load-issuing waves).  "
          "lmhead_gemm_kernel<mode, WM, WNW, WN, KB, SPLIT, NTW>: a workgroup of 64 WM rows by 32 WNW WN "
          "columns, k stages of KB; SPLIT: four more waves issue the loads; NTW: weights read with the nt "
          "policy.  Mode 0 stores logits (the logits launch, and the fused step's probe), 1 keeps the tokens "
          "above the probe's threshold, 2 stores the logits of rows whose candidates overflowed (returns at "
          "once otherwise).", "",
          "## per launch shape (kernel_trace.csv)", ""] + shape_table(perl, lambda n, g: True)
    with open(os.path.join(os.path.dirname(out), "lmhead_b64_b256.md"), "w") as fh:
        fh.write("\n".join(ll) + "\n")


LEGS = ("c2", "verify", "stress", "c0", "c1", "c4", "lmhead", "ref")


def _events_us(fn, n, stream=None):
    """Mean GPU time per call of fn(i) over n back-to-back calls (HIP events
    on the stream the work runs on)."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for i in range(n):
        fn(i)
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / n


def _replay_median_us(graph, n):
    """Median GPU time of one replay of `graph` over n replays, each
    bracketed by HIP events on the stream it replays on (the current one)."""
    import statistics
    import torch
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(st)
        graph.replay()
        b.record(st)
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1000.0 for a, b in ev)


def _capture(fn, n, stream):
    """A hipGraph holding fn(0), ..., fn(n-1), captured on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def sample_leg(L, wl, copies, stream, steps, warmup, median_replays):
    """Sampling steps over `copies` rotating device copies of the workload's
    logits (and bitmask), one step per copy in a graph.  Returns the exact
    `steps`-step wall time per step, the median per step over
    `median_replays` event-timed replays, and the Stage-1 launch time (the
    step's own first launch, HIP events, mean of back-to-back launches)."""
    import time
    import torch
    dev = torch.device("cuda:0")
    B, V = wl.B, wl.V
    x0 = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    if wl.req.bitmask is not None:
        bm0 = torch.from_numpy(wl.req.bitmask.view(np.int32)).to(dev)
        dreqs = [L.DeviceRequests(wl.req).with_bitmask(bm0 if i == 0 else bm0.clone()) for i in range(copies)]
    else:
        d = L.DeviceRequests(wl.req)
        dreqs = [d] * copies
    rng = L.make_rng(0, 0)
    toks = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = L.workspace(B, V, L.SS_BF16)

    def step(i):
        L.ss_sample_step(xs[i % copies], dreqs[i % copies], rng, toks, ws=ws, stream=stream, rng_advance=1)

    # the timed steps: one graph of exactly `steps` steps (step i on copy
    # i mod copies), replayed once, so the steps run back to back with no
    # host call between them; warm-up replays of the same graph first
    timed = _capture(step, steps, stream)
    for _ in range(max(1, -(-warmup // steps))):
        timed.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timed.replay()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    del timed
    full = _capture(step, copies, stream)
    full.replay()
    med_us = _replay_median_us(full, median_replays) / copies
    # Stage 1 alone: ss_tile_topk with the requests is the step's first
    # launch (same grid, listed-token workgroups included)
    cur = torch.cuda.current_stream()
    n1 = max(steps, 50)
    for i in range(copies):
        L.ss_tile_topk(xs[i], 1, dreqs[i], None, ws)
    s1_us = _events_us(lambda i: L.ss_tile_topk(xs[i % copies], 1, dreqs[i % copies], None, ws), n1, cur)
    eager_us = _events_us(lambda i: L.ss_sample_step(xs[i % copies], dreqs[i % copies], rng, toks, ws=ws),
                          n1, cur)
    out = {"step_s": step_s, "median_step_us": med_us, "stage1_us": s1_us, "eager_step_us": eager_us,
           "stage1_launches": n1}
    del full, xs, dreqs
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=16)
    ap.add_argument("--median-replays", type=int, default=200,
                    help="event-timed graph replays behind the median step time")
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma list of workloads to run besides the headline: " + ",".join(LEGS[1:]))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-verify", action="store_true", help="skip the verification latency")
    ap.add_argument("--no-extra", action="store_true", help="run only the headline (and verify, cpu)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run the reads and writes of known size that scale HBM byte counters")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="write the profiles/ summary from the rocprofv3 runs in DIR and exit")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, PROFILE_MD)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the sampling path runs on a single MI355X "
              "(rows shard across GPUs with no communication); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)
    legs = set(x for x in args.legs.split(",") if x)
    if args.no_verify:
        legs.discard("verify")
    if args.no_extra:
        legs &= {"verify"}

    import torch
    from speculative_decoding_verification_stage1_amd import _lib as L
    from speculative_decoding_verification_stage1_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.time()
    wl = W.workload_c2()
    B, V = wl.B, wl.V
    gen_s = time.time() - t_gen
    stream = torch.cuda.Stream()

    # ---- headline: the c2 sampling step, exactly --steps steps timed ----
    h = sample_leg(L, wl, args.copies, stream, args.steps, args.warmup, args.median_replays)
    step_s = h["step_s"]
    tokens_per_s = B / step_s
    e2e_bytes = alg_bytes_per_row(V, PRIOR, NBIAS) * B
    s1_bytes = stage1_bytes_per_row(V, PRIOR, NBIAS) * B
    s1_us = h["stage1_us"]
    s1_gbps = s1_bytes / (s1_us * 1e-6) / 1e9

    result = {
        "metric": "sampled tokens/s and logits GB/s (% HBM peak) at B=256, V=2^18; verify us",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "c2: B=256 V=262144 bf16 logits 2*N(0,1)+10 on 8 ids, grammar bitmask 5% allowed, "
                        "repetition/frequency/presence over 64 prior ids, 16 bias ids, mixed greedy/top-k/"
                        "top-p/min-p; the timed steps in one hipGraph, step i on rotating input copy i mod 16",
            "input_copies": args.copies,
            "global_batch": B, "vocab": V, "tile": L.ss_tile_size(L.SS_BF16), "parallelism": "single-gpu",
        },
        "median_step_us": round(h["median_step_us"], 3),
        "median_replays": args.median_replays,
        "median_tokens_per_s": round(B / (h["median_step_us"] * 1e-6), 1),
        "logits_GBps": round(V * 2 * B / step_s / 1e9, 1),
        "e2e_alg_GBps": round(e2e_bytes / step_s / 1e9, 1),
        "e2e_hbm_frac": round(e2e_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        "stage1_us": round(s1_us, 3),
        "eager_step_us": round(h["eager_step_us"], 3),
        "roofline": {
            "kernel": "stage1_kernel<bf16> (the sampling step's first launch, listed-token workgroups included)",
            "bound": "hbm",
            "achieved": round(s1_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(s1_gbps / HBM_PEAK_GBPS, 4),
            # HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE,
            # scaled by reads and writes of known size
            # (profiles/stage1_bf16_c2.md); None once the kernel sources
            # differ from the ones measured there
            "traffic": recorded_traffic(),
            "alg_bytes_per_launch": s1_bytes,
            "launches_timed": h["stage1_launches"],
        },
        "input_gen_s": round(gen_s, 2),
    }

    if "verify" in legs:
        result.update(verify_measurements(L, W, dev, stream, args))
    if "stress" in legs:
        result["stage1_stress"] = stress_measurements(L, W, stream, h)
    result.update(extra_measurements(args, dev, L, W, stream, legs))
    rr = result.get("read_reference")
    if rr:   # Stage 1 and the whole step against the measured streaming read
        result["stage1_frac_of_read_reference"] = round(result["roofline"]["achieved"] / rr["GBps"], 4)
        result["e2e_frac_of_read_reference"] = round(result["e2e_alg_GBps"] / rr["GBps"], 4)

    # ---- CPU oracle on a bounded sample of the same workload ----
    if not args.no_cpu:
        result.update(cpu_baseline(args, wl, W))

    if args.copy_calibration:
        # HBM counter scale: a streaming read of 1 GiB with the logits'
        # load policy (FETCH_SIZE), and a copy writing 128 MiB (WRITE_SIZE)
        rbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        rout = torch.zeros(2048, dtype=torch.int32, device=dev)
        src = torch.ones(64 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            L.ss_stream_read(rbuf, rout)
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    print(json.dumps(result))


def verify_measurements(L, W, dev, stream, args):
    """c3 verification latency (B=64, gamma=4, V=2^17): bounded, with
    per-request draft counts, and the dense whole-vocabulary variant."""
    import torch
    out = {}
    vw = W.workload_verify()
    G = vw.gamma
    tcopies = 7   # 7 x 80 MiB of target logits: more than the 256 MB last-level cache
    t0d = torch.from_numpy(vw.target.view(np.int16)).to(dev).view(torch.bfloat16)
    ts = [t0d] + [t0d.clone() for _ in range(tcopies - 1)]
    vreq = L.DeviceRequests(vw.req)
    rng = L.make_rng(0, 0)
    d = torch.from_numpy(vw.draft_ids).to(dev)
    q = torch.from_numpy(vw.draft_probs).to(dev)
    vout = torch.zeros((vw.B, G + 1), dtype=torch.int32, device=dev)
    vne = torch.zeros(vw.B, dtype=torch.int32, device=dev)
    vws = L.workspace(vw.B * (G + 1), vw.V, L.SS_BF16)
    nrep = max(20, args.median_replays)

    def timed(fn):
        g = _capture(fn, tcopies, stream)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        mean = _events_us(lambda i: g.replay(), nrep) / tcopies
        med = _replay_median_us(g, nrep) / tcopies
        del g
        return mean, med

    mean, med = timed(lambda i: L.ss_verify_step(ts[i], vw.B, G, vreq, rng, d, q, vout, vne, None, vws,
                                                 stream=stream, rng_advance=1))
    out["verify_us"] = round(mean, 2)
    out["verify_median_us"] = round(med, 2)
    out["verify_config"] = "c3: B=64 gamma=4 V=131072 bf16 target, fp32 draft probs (gathered)"
    out["verify_mean_emitted"] = round(float(vne.float().mean().item()), 3)
    out["verify_acceptance_rate"] = round(float((vne.float() - 1).sum().item()) / (vw.B * G), 4)

    # the same requests with per-request draft counts (seeded, uniform in
    # 0..gamma), passed as inclusive cumulative offsets
    counts = np.random.default_rng(1003).integers(0, G + 1, vw.B)
    cu = torch.from_numpy(np.cumsum(counts).astype(np.int32)).to(dev)
    mean, med = timed(lambda i: L.ss_verify_step_var(ts[i], vw.B, G, vreq, rng, cu, d, q, vout, vne, None, vws,
                                                     stream=stream, rng_advance=1))
    out["verify_var"] = {
        "us": round(mean, 2), "median_us": round(med, 2),
        "draft_counts": "uniform 0..4 per request (seeded), mean %.2f" % float(counts.mean()),
        "mean_emitted": round(float(vne.float().mean().item()), 3),
    }

    # dense variant: whole-vocabulary p, the residual over whole q rows
    # (q rotated too: 7 x 128 MiB), and with no draft probabilities
    qs = [q] + [q.clone() for _ in range(tcopies - 1)]
    dws = L.dense_workspace(vw.B, G, vw.V)
    dense = {}
    for tag, with_q in (("with_q", True), ("no_draft_probs", False)):
        mean, med = timed(lambda i: L.ss_verify_step_dense(ts[i], vw.B, G, vreq, rng, d, qs[i] if with_q else None,
                                                           vout, vne, None, dws, stream=stream, rng_advance=1))
        dense[tag] = {"us": round(mean, 2), "median_us": round(med, 2),
                      "mean_emitted": round(float(vne.float().mean().item()), 3)}
    out["verify_dense"] = dense
    del qs, ts
    torch.cuda.empty_cache()
    return out


def stress_measurements(L, W, stream, head):
    """The tile stage off its usual path, at c2's shape: log-probability
    rows (every logit negative), a 0.1 %-allowed grammar, and more than 128
    list-named tokens in one tile.  Stage-1 launch time and step time, each
    against c2's."""
    import torch
    out = {}
    for kind in W.STRESS_KINDS:
        wl = W.workload_c2_stress(kind)
        r = sample_leg(L, wl, 4, stream, 16, 4, 20)
        out[kind] = {"stage1_us": round(r["stage1_us"], 2),
                     "stage1_vs_c2": round(r["stage1_us"] / head["stage1_us"], 3),
                     "step_us": round(r["median_step_us"], 2),
                     "step_vs_c2": round(r["median_step_us"] / head["median_step_us"], 3)}
        del wl
        torch.cuda.empty_cache()
    out["inputs"] = ("c2 batch with one change each (workloads.workload_c2_stress): log-softmax rows; "
                     "grammar 0.1% allowed; 200 (listed_tile) or 100 (listed_100) prior ids in the first 32768-token tile, "
                     "no grammar; "
                     "4 rotating copies")
    return out


def cpu_baseline(args, wl, W):
    import oracle
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # a one-GPU job's share of the host: 16 cores, whatever the machine has
    cores = max(1, min(avail, 16))
    out = {}
    t0 = time.perf_counter()
    passes = 0
    while True:   # whole passes over all 256 rows until about cpu_seconds of work
        oracle.sample(wl.logits, wl.dtype, wl.req, threads=cores)
        passes += 1
        cpu_s = time.perf_counter() - t0
        if cpu_s >= args.cpu_seconds or passes >= 200:
            break
    out["cpu_baseline"] = {
        "value": round(passes * wl.B / cpu_s, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": f"{passes} passes over all {wl.B} rows of the same workload (oracle.sample, "
                  f"{cores} threads of {avail} usable), {cpu_s:.1f} s",
    }
    sub = W.SampleWorkload(wl.name, wl.dtype, wl.logits[:32], _subset(wl.req, 32))
    t0 = time.perf_counter()
    n1p = 0
    while True:   # one thread, on the first 32 rows (bounded)
        oracle.sample(sub.logits, sub.dtype, sub.req, threads=1)
        n1p += 1
        c1s = time.perf_counter() - t0
        if c1s >= min(3.0, args.cpu_seconds) or n1p >= 50:
            break
    out["cpu_baseline_1thread"] = {"value": round(n1p * 32 / c1s, 2), "unit": "tokens/s", "cores": 1,
                                   "sample": f"{n1p} passes over rows 0-31 of c2, {c1s:.1f} s"}
    return out


def extra_measurements(args, dev, L, W, stream, legs):
    """The other workloads' figures: c0 latency, c1 throughput (cold: 34
    rotating copies > 512 MB), c4 top-k per regime (two-stage threshold and
    radix-bitonic tile selects against the single-program-per-row radix
    select; torch.topk as context), and the streaming-read bandwidth
    reference."""
    import torch
    out = {}
    if "c0" in legs:   # one fp32 row, graph latency (greedy and stochastic)
        c0 = {}
        for greedy in (True, False):
            wl = W.workload_c0(greedy)
            x = torch.from_numpy(wl.logits).to(dev)
            dreq = L.DeviceRequests(wl.req)
            rng = L.make_rng(0, 0)
            tok = torch.zeros(1, dtype=torch.int32, device=dev)
            ws = L.workspace(1, wl.V, L.SS_F32)
            g = _capture(lambda i: L.ss_sample_step(x, dreq, rng, tok, ws=ws, stream=stream, rng_advance=1), 1,
                         stream)
            for _ in range(5):
                g.replay()
            torch.cuda.synchronize()
            gpu_us = _events_us(lambda i: g.replay(), 50)
            t0 = time.perf_counter()
            for _ in range(50):
                g.replay()
                torch.cuda.synchronize()
            sync_us = (time.perf_counter() - t0) / 50 * 1e6
            c0["greedy" if greedy else "stochastic"] = {"graph_replay_us": round(gpu_us, 2),
                                                        "replay_and_sync_us": round(sync_us, 2)}
        out["c0_latency"] = c0
    if "c1" in legs:   # 64 x 131072 bf16, mixed settings
        wl = W.workload_c1()
        B1, V1 = wl.B, wl.V
        ncp = 34
        x1 = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        x1s = [x1] + [x1.clone() for _ in range(ncp - 1)]
        d1 = L.DeviceRequests(wl.req)
        rng = L.make_rng(0, 0)
        tok1 = torch.zeros(B1, dtype=torch.int32, device=dev)
        ws1 = L.workspace(B1, V1, L.SS_BF16)
        g1 = _capture(lambda i: L.ss_sample_step(x1s[i], d1, rng, tok1, ws=ws1, stream=stream, rng_advance=1),
                      ncp, stream)
        g1.replay()
        torch.cuda.synchronize()
        us1 = _replay_median_us(g1, 10) / ncp
        b1 = alg_bytes_per_row(V1, PRIOR, NBIAS, grammar=False) * B1
        out["c1"] = {"step_us": round(us1, 2), "tokens_per_s": round(B1 / (us1 * 1e-6), 1),
                     "alg_GBps": round(b1 / (us1 * 1e-6) / 1e9, 1),
                     "inputs": f"{ncp} rotating copies ({ncp * B1 * V1 * 2 / 2**20:.0f} MiB), median of 10 replays"}
        del x1s, g1
    if "c4" in legs:   # top-k of 512 x 262144 fp32, two regimes
        c4 = {}
        for regime in ("peaked", "flat"):
            tw = W.workload_c4(regime)
            Bk, Vk = tw.logits.shape
            xk = [torch.from_numpy(tw.logits).to(dev)]
            xk.append(xk[0].clone())
            ids = torch.zeros((Bk, tw.k), dtype=torch.int32, device=dev)
            wsk = L.workspace(Bk, Vk, L.SS_F32)
            nbytes = Bk * Vk * 4
            L.ss_topk_step(xk[0], tw.k, ids, ws=wsk)
            two = _events_us(lambda i: L.ss_topk_step(xk[i % 2], tw.k, ids, ws=wsk), 10)
            ids1 = torch.zeros_like(ids)
            L.ss_topk_single_pass(xk[0], tw.k, ids1)
            one = _events_us(lambda i: L.ss_topk_single_pass(xk[i % 2], tw.k, ids1), 3)
            same = bool(torch.equal(ids, ids1))
            idsr = torch.zeros_like(ids)
            L.ss_topk_step_radix(xk[0], tw.k, idsr, ws=wsk)
            rad = _events_us(lambda i: L.ss_topk_step_radix(xk[i % 2], tw.k, idsr, ws=wsk), 10)
            same = same and bool(torch.equal(ids, idsr))
            tt = _events_us(lambda i: torch.topk(xk[i % 2], tw.k, dim=1), 3)
            c4[regime] = {"two_stage_us": round(two, 1), "two_stage_GBps": round(nbytes / (two * 1e-6) / 1e9, 1),
                          "radix_bitonic_us": round(rad, 1),
                          "radix_bitonic_GBps": round(nbytes / (rad * 1e-6) / 1e9, 1),
                          "single_pass_radix_us": round(one, 1),
                          "single_pass_radix_GBps": round(nbytes / (one * 1e-6) / 1e9, 1),
                          "two_stage_speedup_vs_single_pass": round(one / two, 2),
                          "ids_equal": same, "torch_topk_us": round(tt, 1)}
            del xk
        out["c4_topk"] = c4
    if "lmhead" in legs:
        out["lmhead"] = lmhead_measurements(L, W, dev)
    if "ref" in legs:   # the library's streaming read of 1 GiB (four times the last-level cache)
        rbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        rout = torch.zeros(2048, dtype=torch.int32, device=dev)
        L.ss_stream_read(rbuf, rout)
        r_us = _events_us(lambda i: L.ss_stream_read(rbuf, rout), 5)
        out["read_reference"] = {"us": round(r_us, 1), "GBps": round((1 << 30) / (r_us * 1e-6) / 1e9, 1),
                                 "bytes": 1 << 30, "kernel": "ss_stream_read (2048 workgroups, 16-byte nt loads)"}
        del rbuf
    torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0
LMHEAD_SHAPES = ((64, 4096, 131072), (256, 4096, 262144))


def lmhead_measurements(L, W, dev):
    """The LM head fused with sampling, per shape (B, D, V): the fused step,
    the logits launch alone, and the unfused form (logits to memory, then
    the fp32 sampling step), mean of back-to-back launches (HIP events);
    the GEMM's rate against the bf16 matrix-core peak and the weight stream
    against HBM.  The weights (1-2 GiB) exceed the last-level cache, so
    every step streams them from HBM.  torch's bf16 GEMM of the same shape
    (fp32 accumulation, bf16 output) is context."""
    import torch
    res = {}
    for B, D, V in LMHEAD_SHAPES:
        h, w, req = W.lmhead_device_inputs(B, D, V, device=dev)
        dreq = L.DeviceRequests(req)
        rng = L.make_rng(0, 0)
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        ws = L.lmhead_workspace(B, V, device=dev)
        z = torch.empty((B, V), dtype=torch.float32, device=dev)
        ws32 = L.workspace(B, V, L.SS_F32, device=dev)

        def fused(i):
            L.ss_lmhead_sample_step(h, w, dreq, rng, tok, ws=ws, rng_advance=1)

        def logits(i):
            L.ss_lmhead_logits(h, w, z)

        def unfused(i):
            L.ss_lmhead_logits(h, w, z)
            L.ss_sample_step(z, dreq, rng, tok, ws=ws32, rng_advance=1)

        def linear(i):
            torch.nn.functional.linear(h, w)

        for f in (fused, logits, unfused, linear):
            f(0)
            f(1)
        torch.cuda.synchronize()
        n = 10
        t_f = _events_us(fused, n)
        t_l = _events_us(logits, n)
        t_u = _events_us(unfused, n)
        t_t = _events_us(linear, n)
        flops = 2.0 * B * D * V
        wbytes = 2.0 * V * D + 2.0 * B * D
        # the GEMM's roofline: the weight stream at the HBM peak or the
        # products at the bf16 matrix-core peak, whichever takes longer
        t_hbm = wbytes / (HBM_PEAK_GBPS * 1e9) * 1e6
        t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
        t_roof = max(t_hbm, t_mfma)
        res[f"B{B}_D{D}_V{V}"] = {
            "fused_step_us": round(t_f, 1), "logits_only_us": round(t_l, 1), "unfused_step_us": round(t_u, 1),
            "fused_speedup_vs_unfused": round(t_u / t_f, 3),
            "fused_tokens_per_s": round(B / (t_f * 1e-6), 1),
            "roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "roofline_us": round(t_roof, 1),
                         "hbm_us": round(t_hbm, 1), "mfma_us": round(t_mfma, 1),
                         "logits_frac": round(t_roof / t_l, 3), "fused_frac": round(t_roof / t_f, 3)},
            "logits_TFLOPs": round(flops / (t_l * 1e-6) / 1e12, 1),
            "logits_frac_mfma_bf16": round(flops / (t_l * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 3),
            "logits_weight_GBps": round(wbytes / (t_l * 1e-6) / 1e9, 1),
            "logits_frac_hbm": round(wbytes / (t_l * 1e-6) / 1e9 / HBM_PEAK_GBPS, 3),
            "torch_linear_bf16_us": round(t_t, 1),
        }
        del h, w, ws, z, ws32
        torch.cuda.empty_cache()
    return res


def _subset(req, n):
    import dataclasses
    kw = {}
    for f in dataclasses.fields(req):
        v = getattr(req, f.name)
        kw[f.name] = None if v is None else v[:n]
    return type(req)(**kw)


if __name__ == "__main__":
    main()
