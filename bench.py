"""Benchmark of the indexer hot path on one MI355X.

Workload (the batched-decode configuration): 64 sequences, context lengths
uniform in [1024, 32768], FP8 E4M3 queries [64, 64 heads, 128] with per-token
scales, fp32 head weights, FP8 key cache with per-token fp32 scales in 64-row
pages drawn at random from a 40000-page pool, top-2048, fixed logits width
65536. One step = schedule + paged scores + top-k, launched back to back on
one stream (the schedule builder only when the split is kept in a buffer).

Timing: K steps, bracketed by synchronize. The same step captured as a
one-step HIP graph is timed alike and reported beside it.
Each step reads its keys from one of several copies of the page pool in
rotation, so the data a step reads was last touched several steps earlier
(more than the 256 MiB last-level cache ago): the timed region reads keys from
HBM, not from the cache. The scoring kernel's average duration comes from a second pass of
K eager back-to-back launches of the same kernel over the same pool rotation,
between two events on its launch stream (rocprofv3's kernel trace of this
command reports the same kernel's average for cross-checking); a third pass
brackets each launch with its own events for the per-launch minimum.

Also reported: the chunked-prefill workload (16384 rows over 4096 committed
keys, causal (r+1)//4, budget 256e6 B, top-2048) as whole-call time, and the
CPU oracle timed on a bounded sample of the decode workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "mqa_logits_fp8_decode_batched_counters")


def kernel_source_digest():
    h = hashlib.sha256()
    for f in ("mqa_logits.hip", "device_common.h", "internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_indexer_page_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(digest, launch_bytes_key):
    """HBM bytes per scoring-kernel launch from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    path = COUNTER_SUMMARY + ".json"
    try:
        with open(path) as fh:
            prof = json.load(fh)
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_digest") != digest:
        return None
    return prof.get(launch_bytes_key)


def decode_bench(args, torch, idx, synth, wl=2, split=None):
    case = synth.workload(wl, canary=False)
    R, W, k, B = case.R, case.W, case.k, case.B
    split = split or args.split
    if split == "auto":
        split = "in-kernel" if B <= 1024 else "buffer"
    c = case.cache
    log("workload %d: B=%d, sum(len)=%d, pool=%d pages" % (wl, B, int(case.lens.sum()), c.num_pages))
    dev = synth.to_device(case)
    n_sets = max(4, args.pool_copies)
    pools = [dev["kdata"]] + [dev["kdata"].clone() for _ in range(n_sets - 1)]
    scales = [dev["kscale"]] + [dev["kscale"].clone() for _ in range(n_sets - 1)]
    query = idx.make_query(case.dtype, dev["q"], dev["q_scale"], dev["w"])
    kvs = [idx.make_kv_cache(case.dtype, c.page_size, c.num_pages, pools[i], c.page_stride,
                             c.row_stride, scales[i], c.scale_page_stride, c.scale_row_stride)
           for i in range(n_sets)]
    n_ctas = args.ctas or idx.idx_recommended_decode_ctas(R, case.dtype, c.page_size, case.next_n)
    cta = torch.empty(idx.idx_schedule_ints(n_ctas), dtype=torch.int32, device="cuda")
    logits = torch.zeros((R, W), dtype=torch.float32, device="cuda")
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty(R, dtype=torch.int32, device="cuda")
    bt_stride = case.block_tables.shape[1]

    # "buffer": the schedule builder writes the split, the scores read it;
    # "in-kernel": no buffer, each scoring work group computes its own range
    cta_arg = cta if split == "buffer" else None

    def schedule():
        if split == "buffer":
            idx.idx_build_schedule(dev["lens"], B, case.next_n, c.page_size, n_ctas, cta)

    def scores(kv):
        idx.idx_paged_mqa_logits(query, kv, dev["block_tables"], bt_stride, dev["lens"], B,
                                 case.next_n, cta_arg, n_ctas, logits, W)

    def topk():
        idx.idx_topk(logits, W, dev["lens"], B, case.next_n, k, out, cnt)

    def step(kv):
        schedule()
        scores(kv)
        topk()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for kv in kvs:
            step(kv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    # One graph per pool copy; step j replays graph j % n_sets.
    graphs = []
    for kv in kvs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(kv)
        graphs.append(g)
    torch.cuda.synchronize()
    for j in range(args.warmup):
        step(kvs[j % n_sets])
    torch.cuda.synchronize()

    # The step as a caller's stream runs it: its launches back to back. The
    # host submits a step in ~15 us, well under the step's GPU time, so the
    # queue stays ahead of the GPU without a head start.
    K = args.steps
    t0 = time.perf_counter()
    for j in range(K):
        step(kvs[j % n_sets])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / K

    # The same step as a one-step graph of its own, timed alike. Each launch
    # of a graph costs ~5 us of GPU time beyond its kernels here (a graph of
    # four steps costs ~1.3 us per step more than the eager launches), so a
    # caller's graph holding its whole decode step pays it once for all of it.
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(K):
        graphs[j % n_sets].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_graph_ms = (t1 - t0) * 1e3 / K

    # Scoring kernel alone: eager launches on the same stream, same pools in
    # rotation. The average is K back-to-back launches between one pair of
    # events (kernel time plus the dispatch gap, as a kernel trace sees it);
    # the per-launch figures bracket each launch with its own events, which
    # adds the events' own overhead to every launch. A sleep kernel first lets
    # the host queue ahead so no event waits on a launch not yet submitted.
    def host_ahead():
        try:
            torch.cuda._sleep(2_000_000)
        except Exception:
            torch.empty(1 << 28, dtype=torch.uint8, device="cuda").zero_()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host_ahead()
    e0.record()
    for j in range(K):
        scores(kvs[j % n_sets])
    e1.record()
    torch.cuda.synchronize()
    kern_avg_ms = e0.elapsed_time(e1) / K
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    host_ahead()
    for j in range(K):
        kev[j][0].record()
        scores(kvs[j % n_sets])
        kev[j][1].record()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in kev]

    lens = case.lens.astype(int)
    E = [max(0, int(l) - (case.next_n - 1 - j)) for l in lens for j in range(case.next_n)]
    tokens = sum(E)
    fp8 = case.dtype == synth.FP8
    row_bytes = 128 + 4 if fp8 else 64 + 4  # key row + its scale(s)
    kbytes = int(lens.sum()) * row_bytes
    qbytes = R * ((64 * 128 + 4) if fp8 else (64 * 64 + 64 * 4)) + R * 64 * 4
    lbytes = tokens * 4
    launch_bytes = kbytes + qbytes + lbytes
    achieved = launch_bytes / (kern_avg_ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    traffic = traffic_from_profile(digest, "hbm_bytes_per_launch")
    return {
        "tokens": tokens,
        "step_ms": step_ms,
        "step_graph_ms": step_graph_ms,
        "kern_avg_ms": kern_avg_ms,
        "kern_min_ms": min(kern_ms),
        "launch_bytes": launch_bytes,
        "achieved_gbs": achieved,
        "traffic": traffic,
        "n_ctas": n_ctas,
        "split": split,
        "digest": digest,
        "case": case,
    }


def counter_run(args, torch, idx, synth):
    """For rocprofv3 --pmc: a plain copy of known size (the counter's scale
    reference), then eager scoring launches over the pool rotation."""
    copy_bytes = 512 << 20
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    d = decode_bench(args, torch, idx, synth)
    log("counter run: copy of %d bytes, then %d scoring launches of %d algorithmic bytes" % (
        copy_bytes, args.steps, d["launch_bytes"]))


def summarize_counters(fetch_dir, write_dir):
    """Turns the two rocprofv3 --pmc runs of `--counters` (FETCH_SIZE, then
    WRITE_SIZE) into the HBM traffic summary the bench line reads: per-dispatch
    KiB scaled by what the same counter reads for the reference copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under %s" % d)
        vals = {}
        with open(files[0]) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (_, name), v in sorted(vals.items()):
            out.setdefault(name, []).append(v)
        return out

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    # durations of the same dispatches, when the FETCH_SIZE run also traced kernels
    durs = []
    for f in glob.glob(os.path.join(fetch_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "mqa_logits_kernel" in r["Kernel_Name"]:
                    durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    pick = lambda m, frag: next(v for n, v in m.items() if frag in n)
    copy_bytes = 512 << 20
    cf, cw = pick(fetch, "copyBuffer")[0], pick(write, "copyBuffer")[0]
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    sf, sw = pick(fetch, "mqa_logits_kernel"), pick(write, "mqa_logits_kernel")
    kf, kw = sum(sf) / len(sf), sum(sw) / len(sw)
    read_b, write_b = kf * 1024 * fs, kw * 1024 * ws
    import synth
    case = synth.workload(2, canary=False)
    algo = int(case.lens.astype(int).sum()) * (128 + 4 + 4) + case.R * (64 * 128 + 4 + 64 * 4)
    summary = {
        "kernel": "mqa_logits_kernel<FP8, 1 row, 4 tiles>",
        "workload": "batched decode: 64 seqs, lens U[1024,32768], FP8, page 64, 40000-page pool",
        "kernel_source_digest": kernel_source_digest(),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <fetch> -o run -- "
            "python3 -u bench.py --counters --steps 8",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- "
            "python3 -u bench.py --counters --steps 8",
            "python3 bench.py --summarize-counters <fetch> <write>",
        ],
        "reference_copy_bytes": copy_bytes,
        "reference_copy_fetch_kib": cf,
        "reference_copy_write_kib": cw,
        "fetch_scale": fs,
        "write_scale": ws,
        "scoring_fetch_kib_per_launch": kf,
        "scoring_write_kib_per_launch": kw,
        "scoring_launches": len(sf),
        "hbm_read_bytes_per_launch": read_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": read_b + write_b,
        "algorithmic_bytes_per_launch": algo,
    }
    if durs:
        dur = sum(durs) / len(durs)
        summary["traced_us_per_launch"] = dur * 1e6
        summary["hbm_gbs_from_counters"] = (read_b + write_b) / dur / 1e9
    with open(COUNTER_SUMMARY + ".json", "w") as fh:
        json.dump(summary, fh, indent=1)
    with open(COUNTER_SUMMARY + ".md", "w") as fh:
        fh.write("# HBM traffic of the batched-decode scoring launch (rocprofv3 PMC)\n\n")
        fh.write("Commands (repository root, one MI355X; FETCH_SIZE and WRITE_SIZE in separate "
                 "runs):\n\n```\n%s\n```\n\n" % "\n".join(summary["commands"]))
        fh.write("`bench.py --counters` copies a 512 MiB tensor (one `__amd_rocclr_copyBuffer` "
                 "dispatch that must read and write 536,870,912 bytes), then launches the scoring "
                 "kernel over the rotated page pools.\n\n")
        fh.write("| dispatch | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |\n|---|---|---|\n")
        fh.write("| reference copy, 512 MiB | %s | %s |\n" % (f"{cf:,.0f}", f"{cw:,.0f}"))
        fh.write("| scoring kernel (avg of %d) | %s | %s |\n\n" % (
            len(sf), f"{kf:,.0f}", f"{kw:,.0f}"))
        fh.write("Scale factors from the reference copy: reads x%.3f, writes x%.3f. Scoring launch: "
                 "%.1f MB read + %.2f MB written = %.1f MB of HBM traffic against %.1f MB "
                 "algorithmic (%.1f%%). Kernel source digest: `%s`.\n" % (
                     fs, ws, read_b / 1e6, write_b / 1e6, (read_b + write_b) / 1e6, algo / 1e6,
                     100.0 * (read_b + write_b) / algo, summary["kernel_source_digest"]))
        if durs:
            fh.write("\nThe FETCH_SIZE run also traced the dispatches: %.1f us per scoring launch on "
                     "average, so the counted HBM traffic moved at %.0f GB/s (%.1f%% of 8 TB/s).\n" % (
                         summary["traced_us_per_launch"], summary["hbm_gbs_from_counters"],
                         summary["hbm_gbs_from_counters"] / 80.0))
    log("wrote %s.{json,md}: %.1f MB per launch (%.1f MB algorithmic)" % (
        COUNTER_SUMMARY, (read_b + write_b) / 1e6, algo / 1e6))


def prefill_bench(args, torch, idx, synth):
    case = synth.workload(4, canary=False)
    T, W, k = case.T, case.W, case.k
    log("workload 4: T=%d, W=%d, budget=%d" % (T, W, case.budget_bytes))
    dev = synth.to_device(case)
    c = case.cache
    query = idx.make_query(case.dtype, dev["q"], dev["q_scale"], dev["w"])
    kv = idx.make_kv_cache(case.dtype, c.page_size, c.num_pages, dev["kdata"], c.page_stride,
                           c.row_stride, dev["kscale"], c.scale_page_stride, c.scale_row_stride)
    sb = idx.idx_prefill_scratch_bytes(T, W, case.budget_bytes)
    si = idx.idx_prefill_schedule_ints(T, W, case.budget_bytes)
    scratch = torch.empty(sb // 4, dtype=torch.float32, device="cuda")
    cta = torch.empty(si, dtype=torch.int32, device="cuda")
    out = torch.empty((T, k), dtype=torch.int32, device="cuda")

    def call():
        idx.idx_prefill_chunked_topk(query, kv, dev["block_table"], dev["visible_end"], T, W,
                                     case.budget_bytes, k, 0, scratch, sb, cta, si, out)

    for _ in range(2):
        call()
    torch.cuda.synchronize()
    n = max(20, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    import numpy as np
    ve = case.visible_end.astype(np.int64)
    pairs = int(ve.sum())
    flops = 2.0 * pairs * 64 * 128
    # rows seeing at most k keys select every one of them, so the call does
    # not score them: the flops the selection needs are those of the others
    needed = 2.0 * int(ve[ve > k].sum()) * 64 * 128
    return {"ms_per_call": ms, "pairs": pairs, "flops": flops, "flops_needed": needed,
            "rows_scored": int((ve > k).sum()),
            "tflops_whole_call": needed / (ms * 1e-3) / 1e12}


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "prefill_logits_fp8_chunked_mfma_counters")
FP8_MFMA_FLOPS = 16 * 16 * 128 * 2  # one v_mfma_f32_16x16x128_f8f6f4


def prefill_source_digest():
    h = hashlib.sha256()
    for f in ("prefill.hip", "device_common.h", "internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_indexer_page_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def summarize_trace(trace_dir, out_md, title, command, scoring_groups=None):
    """A kernel-trace summary (rocprofv3 --kernel-trace --stats, csv) as
    markdown: per-kernel calls and durations, and, when scoring_groups is
    given as [(label, first, count), ...], the average duration of those
    dispatches of the decode scoring kernel in launch order."""
    import csv
    import glob

    def rows(pattern):
        files = glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True)
        if not files:
            raise SystemExit("no %s under %s" % (pattern, trace_dir))
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))

    def short(name):
        name = name.replace("void ", "").replace("idx::(anonymous namespace)::", "")
        return name if len(name) <= 72 else name[:69] + "..."

    stats = rows("*kernel_stats.csv")
    lines = ["# " + title, "", "Command (repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %s |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, r["Percentage"]))
    if scoring_groups:
        trace = rows("*kernel_trace.csv")
        sc = [int(t["End_Timestamp"]) - int(t["Start_Timestamp"]) for t in trace
              if "mqa_logits_kernel" in t["Kernel_Name"]]
        lines += ["", "Decode scoring dispatches in launch order, grouped as bench.py issues them:", "",
                  "| group | dispatches | avg us |", "|---|---|---|"]
        for label, first, count in scoring_groups:
            part = sc[first:first + count]
            if part:
                lines.append("| %s | %d | %.2f |" % (label, len(part), sum(part) / len(part) / 1e3))
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log("wrote " + out_md)


PREFILL_PMC_PASSES = (
    # rocprofv3 collects one pass per run: at most 8 SQ and 2 GRBM counters each
    "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU "
    "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE",
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_SCA "
    "SQ_WAIT_INST_LDS SQ_WAVES GRBM_GUI_ACTIVE",
)
N_XCD = 8     # GRBM_GUI_ACTIVE is summed over the eight XCDs
N_SIMD = 1024  # 256 CUs x 4 SIMDs


def summarize_mfma(pmc_dirs):
    """Counters of the prefill scoring kernel from rocprofv3 runs of
    `--prefill-counters`, one per counter pass (PREFILL_PMC_PASSES, each with
    --kernel-trace), matched by the order of the prefill dispatches: FP8 flops
    per dispatch = MFMA instructions x 16*16*128*2 over the traced duration,
    the engine clock from GRBM_GUI_ACTIVE, and per SIMD the MFMA busy share
    and VALU / LDS / SALU instructions per MFMA."""
    import csv
    import glob

    def one(d, pattern):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not files:
            raise SystemExit("no %s under %s" % (pattern, d))
        with open(files[0]) as fh:
            return list(csv.DictReader(fh))

    merged = None
    for d in pmc_dirs:
        cnt = {}
        for r in one(d, "*counter_collection.csv"):
            if "prefill_logits_kernel" not in r["Kernel_Name"]:
                continue
            e = cnt.setdefault(int(r["Dispatch_Id"]), {})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        dur = {}
        for r in one(d, "*kernel_trace.csv"):
            if "prefill_logits_kernel" in r["Kernel_Name"]:
                dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        rows = [dict(cnt[i], us=dur[i] * 1e6, chunk=n % 2) for n, i in enumerate(sorted(cnt)) if i in dur]
        if merged is None:
            merged = rows
        else:
            if len(rows) != len(merged):
                raise SystemExit("%s has %d prefill dispatches, the first run %d" % (d, len(rows), len(merged)))
            for a, b in zip(merged, rows):
                a.update({k: v for k, v in b.items() if k not in ("us", "chunk")})
    big = merged
    for r in big:
        r["tflops"] = r.get("SQ_INSTS_MFMA", 0.0) * FP8_MFMA_FLOPS / (r["us"] * 1e-6) / 1e12
    tot = lambda key, rows=big: sum(r.get(key, 0.0) for r in rows)
    agg_tflops = tot("SQ_INSTS_MFMA") * FP8_MFMA_FLOPS / (tot("us") * 1e-6) / 1e12
    busy_frac = tot("SQ_VALU_MFMA_BUSY_CYCLES") / (N_SIMD * tot("us") * 1e-6 * 2.4e9)

    def derived(rows):
        us = tot("us", rows)
        cycles = tot("GRBM_GUI_ACTIVE", rows) / N_XCD  # engine cycles of the dispatches
        mfma = tot("SQ_INSTS_MFMA", rows)
        valu = tot("SQ_INSTS_VALU", rows) - mfma  # SQ_INSTS_VALU counts the MFMAs too
        return {
            "us": us,
            "clock_ghz": cycles / (us * 1e-6) / 1e9 if us else 0.0,
            "fp8_tflops": mfma * FP8_MFMA_FLOPS / (us * 1e-6) / 1e12 if us else 0.0,
            # one 16x16x128 FP8 MFMA keeps its SIMD's matrix core 32 cycles
            "mfma_busy_frac": 32.0 * mfma / (N_SIMD * cycles) if cycles else 0.0,
            "valu_per_mfma": valu / mfma if mfma else 0.0,
            "lds_per_mfma": tot("SQ_INSTS_LDS", rows) / mfma if mfma else 0.0,
            "salu_per_mfma": tot("SQ_INSTS_SALU", rows) / mfma if mfma else 0.0,
            # quad-cycles summed over waves, as a share of SIMD cycles
            "valu_active_frac": 4.0 * tot("SQ_ACTIVE_INST_VALU", rows) / (N_SIMD * cycles) if cycles else 0.0,
            "lds_bank_conflicts_per_lds_inst": tot("SQ_LDS_BANK_CONFLICT", rows) / tot("SQ_INSTS_LDS", rows)
            if tot("SQ_INSTS_LDS", rows) else 0.0,
            # a wave's alive time over its dispatch's duration, averaged
            "wave_alive_frac": 4.0 * tot("SQ_WAVE_CYCLES", rows) / tot("SQ_WAVES", rows) / (cycles / len(rows))
            if tot("SQ_WAVES", rows) and cycles else 0.0,
        }

    per_chunk = {c: derived([r for r in big if r["chunk"] == c]) for c in (0, 1)}
    summary = {
        "kernel": "prefill_logits_kernel<FP8, 4 tiles> (both chunks: 8192 + 8192 rows)",
        "workload": "chunked prefill: 16384 rows over 4096 keys, causal (r+1)//4, page 64",
        "kernel_source_digest": prefill_source_digest(),
        "commands": ["rocprofv3 --pmc %s --kernel-trace --output-format csv -d <dir%d> -o run -- "
                     "python3 -u bench.py --prefill-counters" % (c, n + 1)
                     for n, c in enumerate(PREFILL_PMC_PASSES)] +
                    ["python3 bench.py --summarize-mfma %s" % " ".join(
                        "<dir%d>" % (n + 1) for n in range(len(PREFILL_PMC_PASSES)))],
        "dispatches": big,
        "us_per_dispatch": tot("us") / len(big),
        "fp8_tflops": agg_tflops,
        "fp8_mfma_frac": agg_tflops / FP8_MFMA_PEAK_TFLOPS,
        "mfma_busy_frac_at_2p4ghz": busy_frac,
        "per_chunk": {"short rows (0-2048 keys)": per_chunk[0], "long rows (2048-4096 keys)": per_chunk[1]},
    }
    with open(MFMA_SUMMARY + ".json", "w") as fh:
        json.dump(summary, fh, indent=1)
    names = [n for n in PREFILL_PMC_PASSES[0].split() + PREFILL_PMC_PASSES[1].split()]
    names = [n for i, n in enumerate(names) if n not in names[:i]]
    with open(MFMA_SUMMARY + ".md", "w") as fh:
        fh.write("# Pipe use of the chunked-prefill scoring kernel (rocprofv3 PMC)\n\n")
        fh.write("Commands (repository root, one MI355X; one counter pass per run):\n\n```\n%s\n```\n\n" %
                 "\n".join(summary["commands"]))
        fh.write("`bench.py --prefill-counters` runs the 16384-row chunked prefill call (budget 256e6 B: "
                 "two chunks of 8192 rows; the first sees 0-2048 keys per row, the second 2048-4096). "
                 "Counters are summed over all XCDs and SIMDs; the runs' dispatches are matched in "
                 "order.\n\n")
        fh.write("| dispatch | chunk | traced us | FP8 TFLOP/s | " + " | ".join(names) + " |\n")
        fh.write("|---" * (4 + len(names)) + "|\n")
        for n, r in enumerate(big):
            fh.write("| %d | %d | %.1f | %.0f | %s |\n" % (
                n, r["chunk"], r["us"], r["tflops"],
                " | ".join(f"{r.get(k, 0.0):,.0f}" for k in names)))
        fh.write("\n## Derived, per chunk\n\n| | short rows | long rows |\n|---|---|---|\n")
        labels = [("traced us (sum)", "us", "%.1f"), ("engine clock, GHz (GRBM_GUI_ACTIVE / 8 / time)", "clock_ghz", "%.2f"),
                  ("FP8 TFLOP/s", "fp8_tflops", "%.0f"),
                  ("MFMA busy share of SIMD cycles (32 cycles per MFMA)", "mfma_busy_frac", "%.3f"),
                  ("VALU instructions per MFMA (SQ_INSTS_VALU less the MFMAs)", "valu_per_mfma", "%.2f"),
                  ("VALU active share of SIMD cycles (4 x SQ_ACTIVE_INST_VALU)", "valu_active_frac", "%.3f"),
                  ("LDS instructions per MFMA", "lds_per_mfma", "%.3f"),
                  ("SALU instructions per MFMA", "salu_per_mfma", "%.2f"),
                  ("LDS bank conflicts per LDS instruction", "lds_bank_conflicts_per_lds_inst", "%.3f"),
                  ("wave-alive share of the dispatch (4 x SQ_WAVE_CYCLES / SQ_WAVES / cycles)", "wave_alive_frac", "%.3f")]
        for lab, key, fmt in labels:
            fh.write("| %s | %s | %s |\n" % (lab, fmt % per_chunk[0][key], fmt % per_chunk[1][key]))
        fh.write("\nAll dispatches: %.0f TFLOP/s = %.1f%% of the 5.0 PFLOP/s dense FP8 peak. Kernel source "
                 "digest: `%s`.\n" % (agg_tflops, 100 * agg_tflops / FP8_MFMA_PEAK_TFLOPS,
                                       summary["kernel_source_digest"]))
    log("wrote " + MFMA_SUMMARY + ".md")
    print(json.dumps({k: v for k, v in summary.items() if k != "dispatches"}, indent=1))


def prefill_counter_run(args, torch, idx, synth):
    """For rocprofv3 --pmc: three eager chunked-prefill calls."""
    args.steps = 12
    prefill_bench(args, torch, idx, synth)


def kv_write_bench(args, torch, idx, synth):
    """K-cache writer: 65536 new bf16 key rows quantized to FP8 and scattered
    over a 1024-page pool of 64-row pages (rows in a random slot order)."""
    import numpy as np
    P, pages, N = 64, 1024, 65536
    cache = synth._alloc_cache(synth.FP8, pages, P, 128, None, "separate", False)
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((N, 128)).astype(np.float32)).to(torch.bfloat16)
    k = k.cuda()
    slots = torch.from_numpy(rng.permutation(pages * P)[:N].astype(np.int64)).cuda()
    data = torch.from_numpy(cache.data).cuda()
    scale = torch.from_numpy(cache.scale).cuda()
    kv = idx.make_kv_cache(synth.FP8, P, pages, data, cache.page_stride, cache.row_stride, scale,
                           cache.scale_page_stride, cache.scale_row_stride)

    def call():
        idx.idx_kv_cache_write(k, idx.IDX_KIN_BF16, 128, N, slots, kv)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = N * (128 * 2 + 128 + 4 + 8)  # bf16 row in, FP8 row + scale out, slot
    return {"workload": "K-cache write: 65536 bf16 rows -> FP8 + fp32 scale, page 64, "
                        "random slots", "rows": N, "us_per_call": ms * 1e3,
            "rows_per_s": N / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "achieved_gbs": nbytes / (ms * 1e-3) / 1e9}


def q_quant_bench(args, torch, idx, R_decode):
    """Query quantization with the weight fold: bf16 query rows of 64 x 128
    to FP8 codes with the row scale folded into the weights, for the decode
    batch's rows and for a 16384-row prefill batch."""
    import numpy as np
    rng = np.random.default_rng(4)
    res = []
    for R in (R_decode, 16384):
        x = torch.from_numpy(rng.standard_normal((R, 8192), dtype=np.float32)).to(torch.bfloat16)
        x = x.cuda()
        w = torch.randn((R, 64), dtype=torch.float32, device="cuda")
        q = torch.empty((R, 8192), dtype=torch.uint8, device="cuda")
        wo = torch.empty((R, 64), dtype=torch.float32, device="cuda")
        out = idx.make_query(idx.IDX_FP8_E4M3, q, None, wo)

        def call():
            idx.idx_quantize_query(x, idx.IDX_KIN_BF16, 8192, R, w, 0.0883883, out)

        for _ in range(3):
            call()
        torch.cuda.synchronize()
        n = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        nbytes = R * (8192 * 2 + 8192 + 64 * 4 * 2)  # bf16 in, FP8 out, weights in + out
        res.append({"rows": R, "us_per_call": ms * 1e3, "algorithmic_bytes": nbytes,
                    "achieved_gbs": nbytes / (ms * 1e-3) / 1e9})
    return {"workload": "query quantization: bf16 [R][64][128] -> FP8 with the row scale "
                        "folded into the weights", "runs": res}


def sparse_mla_bench(args, torch, idx, synth):
    """Sparse attention over the decode batch's selection: 64 rows, 2048
    listed tokens each in ascending token order, as the top-k writes them
    (512-dim bf16 latent rows, page 64), 64 heads. Calls
    rotate over four copies of the latent cache (each call's 134 MB of rows
    was last touched three calls earlier, beyond the 256 MiB last-level
    cache), timed back to back between two events."""
    import numpy as np
    rng = np.random.default_rng(9)
    lens = rng.integers(2048, 32768 + 1, size=64)
    # lists in ascending token order, as idx_topk writes them
    case = synth.mla_case(lens, next_n=1, P=64, k=2048, seed=10, ascending=True)
    R, k = case.R, case.k
    q = torch.from_numpy(case.q.view(np.int16)).cuda()
    data = torch.from_numpy(case.data).cuda()
    copies = [data] + [data.clone() for _ in range(3)]
    bt = torch.from_numpy(case.block_tables).cuda()
    ind = torch.from_numpy(case.indices).cuda()
    tl = torch.from_numpy(case.topk_lens).cuda()
    out = torch.empty((R, 64, 512), dtype=torch.int16, device="cuda")
    lse = torch.empty((R, 64), dtype=torch.float32, device="cuda")
    wsb = idx.idx_sparse_mla_workspace_size(R, k)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device="cuda")
    kvs = [idx.make_mla_cache(case.page_size, case.num_pages, d, case.page_stride,
                              case.row_stride) for d in copies]

    def call(j):
        idx.idx_sparse_mla_decode(q, kvs[j % len(kvs)], bt, case.block_tables.shape[1], R, 1, ind,
                                  tl, k, 0.0442, out, lse, ws, wsb)

    for j in range(4):
        call(j)
    torch.cuda.synchronize()
    n = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for j in range(n):
        call(j)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    listed = int(case.topk_lens.sum())
    nbytes = listed * 1024 + R * 64 * 512 * 2 * 2 + R * k * 4  # rows, q + out, lists
    flops = 2.0 * 2 * listed * 64 * 512
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "sparse attention over the selection: 64 rows x 2048 listed tokens, "
                        "64 heads, 512-dim bf16 latent rows, page 64",
            "us_per_call": ms * 1e3, "algorithmic_bytes": nbytes,
            "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "bf16_tflops": flops / (ms * 1e-3) / 1e12, "workspace_bytes": wsb}


def host_cpu():
    """The host the CPU baseline ran on: logical CPUs, the ones this process
    may use, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(case, budget_s):
    """The CPU oracle on a bounded sample of the decode workload: groups of
    rows in a fixed random order, cycling over the workload's rows, until
    about budget_s seconds of work are done (a pass over all rows can be far
    shorter than that, and a longer sample steadies the rate)."""
    import numpy as np

    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import oracle_cache

    rows_all = np.arange(case.R)
    rng = np.random.default_rng(0)
    order = rng.permutation(rows_all)
    cache = oracle_cache(case)
    done, tokens, elapsed = [], 0, 0.0
    t0 = time.perf_counter()
    chunk = max(oracle.threads(), 1)
    i = 0
    while elapsed < budget_s:
        rows = order[np.arange(i, i + chunk) % len(order)]
        lg, E = oracle.decode_logits(case.dtype, case.q, case.q_scale, case.w, case.H, case.D,
                                     cache, case.block_tables, case.lens, case.next_n, rows,
                                     case.W)
        oracle.topk_rows_f32(lg.astype(np.float32), E, case.k)
        tokens += int(E.sum())
        done.extend(rows.tolist())
        i += chunk
        elapsed = time.perf_counter() - t0
    return {
        "value": tokens / elapsed,
        "unit": "tokens/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "host": host_cpu(),
        "sample": "%d row evaluations cycling over the %d decode rows (%d scored tokens, "
                  "logits + top-k), %.1f s" % (len(done), case.R, tokens, elapsed),
    }


CEILINGS_MD = os.path.join(ROOT, "profiles", "ceilings_mi355x.md")


def ceilings(torch, write_dir=None):
    """Roofline ceilings measured on this GPU with the kernels of
    sparse_attention_indexer_page_amd/ceilings: the paged streaming-read rate
    (random key pages, the scoring kernel's MFMA-ordered loads and linear 1 KB
    loads) and the FP8 MFMA rate alone, with the scoring epilogue, and the
    epilogue alone. Writes profiles/ceilings_mi355x.md."""
    import ctypes
    import numpy as np
    from sparse_attention_indexer_page_amd import build
    if not os.path.exists(build.CEILINGS_LIB):
        build.build_ceilings()
    lib = ctypes.CDLL(build.CEILINGS_LIB)
    P = ctypes.c_void_p
    lib.ceil_stream_pages.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
    lib.ceil_mfma_epilogue.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn, reps=4):
        best = 1e30
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = fn()
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise SystemExit("ceiling kernel launch failed: %d" % rc)
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        return best

    res = {"stream": [], "mfma": []}
    pool_bytes = 2 << 30  # 8x the 256 MiB last-level cache; each page read once
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    out = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(7)
    for kind, (rows, stride) in ((0, (32, 144)), (1, (64, 128))):
        page = rows * stride
        n_pages = pool_bytes // page // 4  # 512 MiB of pages touched per pass
        for waves in (1024, 2048):
            ppw = (n_pages // waves) // 2 * 2
            pages = torch.from_numpy(rng.permutation(n_pages)[:waves * ppw].astype(np.int32)).cuda()
            for linear in (0, 1):
                t = timed(lambda: lib.ceil_stream_pages(pool.data_ptr(), pages.data_ptr(), ppw, waves,
                                                        kind, linear, out.data_ptr(), stream))
                gbs = waves * ppw * page / t / 1e9
                res["stream"].append({"page": "%d x %d B" % (rows, stride), "waves": waves,
                                      "loads": "linear 1 KB" if linear else "MFMA order (16 rows x 64 B)",
                                      "us": t * 1e6, "gbs": gbs, "frac_of_8tbs": gbs / HBM_PEAK_GBS})
                log("ceiling stream %s, %d waves, %s: %.0f GB/s" % (
                    res["stream"][-1]["page"], waves, res["stream"][-1]["loads"], gbs))
    del pool
    # FP8 operands: a low-entropy pattern, and random finite E4M3 codes (what
    # quantized keys and queries look like; they draw more power and the
    # clock drops, so this is the ceiling the scoring kernels face)
    low = (np.arange(1024, dtype=np.int64) * 2654435761 & 0x3C3C3C3C).astype(np.int32)
    codes = rng.integers(0, 256, size=4096, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] -= 1  # no NaN codes
    operands = (("low-entropy pattern", low), ("random FP8 codes", codes.view(np.int32)))
    fout = torch.empty(256 * 1024, dtype=torch.float32, device="cuda")
    iters = 4000
    for (data, host), threads in [(o, t) for o in operands for t in (256, 512, 1024)]:
        inp = torch.from_numpy(np.ascontiguousarray(host)).cuda()
        row = {"operands": data, "waves_per_simd": threads // 256}
        for mode, name in ((0, "mfma"), (1, "epilogue"), (2, "mfma_and_epilogue")):
            t = timed(lambda: lib.ceil_mfma_epilogue(inp.data_ptr(), fout.data_ptr(), iters, mode, 256,
                                                     threads, stream), reps=3)
            waves = 256 * threads // 64
            row[name + "_us"] = t * 1e6
            if mode != 1:  # 8 MFMAs of 65536 flops per wave per iteration
                row[name + "_tflops"] = waves * iters * 8 * 65536 / t / 1e12
            else:          # 32 scores (2*relu + multiply-add) per lane per iteration
                row["epilogue_gscores_per_s"] = waves * 64 * iters * 32 / t / 1e9
        row["mfma_and_epilogue_frac_of_5pf"] = row["mfma_and_epilogue_tflops"] / FP8_MFMA_PEAK_TFLOPS
        row["mfma_frac_of_5pf"] = row["mfma_tflops"] / FP8_MFMA_PEAK_TFLOPS
        res["mfma"].append(row)
        log("ceiling MFMA, %s, %d waves/SIMD: MFMA alone %.0f TF, with the epilogue %.0f TF (%.1f%% of 5 PF)" % (
            data, row["waves_per_simd"], row["mfma_tflops"], row["mfma_and_epilogue_tflops"],
            100 * row["mfma_and_epilogue_frac_of_5pf"]))
    cmd = "python3 bench.py --ceilings"
    lines = ["# Roofline ceilings measured on the MI355X", "", "Command (repository root, one MI355X):", "",
             "```", cmd, "```", "",
             "Kernels: `sparse_attention_indexer_page_amd/ceilings/ceilings.hip`.", "",
             "## Paged streaming read (random pages, each read once, 512 MiB per pass, one page ahead per wave)",
             "", "| page | waves | loads | us | GB/s | of 8 TB/s |", "|---|---|---|---|---|---|"]
    for r in res["stream"]:
        lines.append("| %s | %d | %s | %.1f | %.0f | %.1f%% |" % (r["page"], r["waves"], r["loads"], r["us"],
                                                               r["gbs"], 100 * r["frac_of_8tbs"]))
    lines += ["", "## FP8 MFMA (16x16x128) and the scoring epilogue (256 work groups)", "",
              "Per wave and iteration: 8 MFMAs (mfma), the epilogue of 32 scores per lane: s + |s| and a "
              "multiply-add each (epilogue), or both in the scoring kernel's proportion (8 VALU ops per MFMA).",
              "", "| operands | waves/SIMD | MFMA alone TF/s | epilogue alone G scores/s | both: TF/s | both: of 5 PF |",
              "|---|---|---|---|---|---|"]
    for r in res["mfma"]:
        lines.append("| %s | %d | %.0f | %.0f | %.0f | %.1f%% |" % (
            r["operands"], r["waves_per_simd"], r["mfma_tflops"], r["epilogue_gscores_per_s"], r["mfma_and_epilogue_tflops"],
            100 * r["mfma_and_epilogue_frac_of_5pf"]))
    out_md = os.path.join(write_dir, os.path.basename(CEILINGS_MD)) if write_dir else CEILINGS_MD
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log("wrote " + out_md)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--ctas", type=int, default=0, help="schedule work groups (0: recommended)")
    ap.add_argument("--pool-copies", type=int, default=4)
    ap.add_argument("--split", choices=("auto", "buffer", "in-kernel"), default="auto",
                    help="decode work split: schedule buffer or computed in the scoring kernel "
                         "(auto: in-kernel for B <= 1024)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--prefill-counters", action="store_true",
                    help="eager prefill calls only (for rocprofv3 --pmc)")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR", nargs="+",
                    help="write the profiles/ MFMA summary from a --prefill-counters PMC run")
    ap.add_argument("--counters", action="store_true",
                    help="only a reference copy + scoring launches, for rocprofv3 --pmc runs")
    ap.add_argument("--sparse-attention-only", action="store_true",
                    help="time only the sparse attention over the selection (one JSON line)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="(the default run times every decode workload; kept for the profile commands)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the streaming-read and MFMA ceilings (writes profiles/ceilings_mi355x.md)")
    ap.add_argument("--write-dir", default=None,
                    help="write generated summaries here instead of profiles/")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the profiles/ kernel-trace summary of a --kernel-trace --stats run")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ traffic summary from two --counters PMC runs")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        d = args.summarize_trace
        if args.all_workloads:
            summarize_trace(d, os.path.join(ROOT, "profiles", "kernels_all_decode_workloads.md"),
                            "Kernel trace of bench.py --all-workloads: batched decode (FP8, 1 row, "
                            "64-row pages: mqa_logits_kernel<1, 1, 4>), single-sequence decode (same "
                            "instance), MTP decode (FP8, 2 rows, 32-row pages: <1, 2, 2>), MXFP4 decode "
                            "(<2, 1, 4>), and the rest of the bench",
                            "rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                            "python3 -u bench.py --all-workloads --steps 20 --warmup 5 --no-cpu-baseline\n"
                            "python3 bench.py --all-workloads --summarize-trace <dir>")
        elif args.sparse_attention_only:
            summarize_trace(d, os.path.join(ROOT, "profiles", "sparse_mla_decode_64x2048_kernel_trace.md"),
                            "Kernel trace of the sparse attention over the selection: 64 rows x 2048 "
                            "listed tokens, 64 heads, 512-dim bf16 latent rows, page 64",
                            "rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                            "python3 -u bench.py --sparse-attention-only\n"
                            "python3 bench.py --sparse-attention-only --summarize-trace <dir>")
        else:
            # per decode run: 4 eager steps, warmup steps, timed steps, 4 graph
            # warmup replays, timed graph replays, back-to-back scoring
            # launches, bracketed scoring launches
            n, w = args.steps, args.warmup
            groups = []
            for i, run in enumerate(("in-kernel split", "schedule buffer")):
                base = i * (8 + w + 4 * n)
                groups += [(run + ": timed steps (eager launches)", base + 4 + w, n),
                           (run + ": timed one-step graph replays", base + 8 + w + n, n),
                           (run + ": back-to-back scoring launches (the bench's average)",
                            base + 8 + w + 2 * n, n),
                           (run + ": scoring launches, each bracketed by events",
                            base + 8 + w + 3 * n, n)]
            summarize_trace(d, os.path.join(ROOT, "profiles", "kernels_decode_batched_and_prefill_chunked.md"),
                            "Kernel trace of bench.py: batched decode (64 seqs, FP8, page 64, top-2048, "
                            "eager steps and graph replays; with and without the schedule buffer), "
                            "chunked prefill (16384 rows x 4096 keys, 2 chunks), K-cache write, query "
                            "quantization, sparse attention",
                            "rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                            "python3 -u bench.py --steps %d --warmup %d --no-cpu-baseline\n"
                            "python3 bench.py --steps %d --warmup %d --summarize-trace <dir>" % (n, w, n, w),
                            groups)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(decode shards by sequence and prefill by query row, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import sparse_attention_indexer_page_amd as idx
    from sparse_attention_indexer_page_amd import build

    build.ensure_built()  # rebuilds when a source changed since the last build
    idx.load()
    torch.cuda.set_device(0)

    if args.ceilings:
        ceilings(torch, args.write_dir)
        return
    if args.counters:
        counter_run(args, torch, idx, synth)
        return
    if args.prefill_counters:
        prefill_counter_run(args, torch, idx, synth)
        return
    if args.sparse_attention_only:
        print(json.dumps(sparse_mla_bench(args, torch, idx, synth)), flush=True)
        return
    d = decode_bench(args, torch, idx, synth)
    log("decode (%s split): step %.3f ms (one-step graph %.3f ms), scoring kernel %.3f ms avg "
        "(%.3f min), %.0f GB/s" % (d["split"], d["step_ms"], d["step_graph_ms"], d["kern_avg_ms"],
                                   d["kern_min_ms"], d["achieved_gbs"]))
    alt = None
    if d["split"] == "in-kernel" and not args.no_prefill:
        alt = decode_bench(args, torch, idx, synth, split="buffer")
        log("decode (buffer split): step %.3f ms, scoring kernel %.3f ms avg" % (
            alt["step_ms"], alt["kern_avg_ms"]))
    pre = None if args.no_prefill else prefill_bench(args, torch, idx, synth)
    if pre:
        log("prefill: %.3f ms per chunked call, %.1f TFLOP/s whole call" % (
            pre["ms_per_call"], pre["tflops_whole_call"]))
    kvw = None if args.no_prefill else kv_write_bench(args, torch, idx, synth)
    if kvw:
        log("kv write: %.1f us per %d rows, %.0f GB/s" % (kvw["us_per_call"], kvw["rows"],
                                                         kvw["achieved_gbs"]))
    qq = None
    if not args.no_prefill:
        qq = q_quant_bench(args, torch, idx, d["case"].R)
        for r in qq["runs"]:
            log("query quantization: %.1f us per %d rows, %.0f GB/s" % (
                r["us_per_call"], r["rows"], r["achieved_gbs"]))
    mla = None
    if not args.no_prefill:
        mla = sparse_mla_bench(args, torch, idx, synth)
        log("sparse attention: %.1f us per call, %.0f GB/s, %.1f TFLOP/s bf16" % (
            mla["us_per_call"], mla["achieved_gbs"], mla["bf16_tflops"]))
    others = []
    if not args.no_prefill:
        for wl in (1, 3, 5):
            o = decode_bench(args, torch, idx, synth, wl)
            log("workload %d: step %.3f ms, scoring kernel %.3f ms avg, %.0f GB/s (%.1f%% of peak)" % (
                wl, o["step_ms"], o["kern_avg_ms"], o["achieved_gbs"],
                100.0 * o["achieved_gbs"] / HBM_PEAK_GBS))
            others.append({"workload": synth.WORKLOADS[wl], "tokens": o["tokens"],
                           "ms_per_step": o["step_ms"], "ms_per_step_graph": o["step_graph_ms"],
                           "scoring_kernel_us": o["kern_avg_ms"] * 1e3,
                           "tokens_per_s": o["tokens"] / (o["step_ms"] * 1e-3),
                           "algorithmic_bytes_per_launch": o["launch_bytes"],
                           "achieved_gbs": o["achieved_gbs"],
                           "hbm_frac": o["achieved_gbs"] / HBM_PEAK_GBS,
                           "n_ctas": o["n_ctas"]})
    cpu = None if args.no_cpu_baseline else cpu_baseline(d["case"], args.cpu_budget_s)

    value = d["tokens"] / (d["step_ms"] * 1e-3)
    line = {
        "metric": "indexer tokens scored/sec (decode step: schedule + paged FP8 MQA scores + top-k)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d["step_ms"],
        "ms_per_step_one_step_graph": d["step_graph_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": "batched decode: 64 seqs, lens U[1024,32768], next_n 1, FP8 q/K + "
                        "per-token fp32 scales, page 64, 40000-page pool, top-2048, "
                        "launches back to back on one stream, logits [64, 65536]",
            "global_batch": 64,
            "seq_len": "U[1024,32768]",
            "parallelism": "single GPU",
            "n_ctas": d["n_ctas"],
            "split": d["split"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": d["achieved_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": d["achieved_gbs"] / HBM_PEAK_GBS,
            "traffic": d["traffic"],
            "kernel": "mqa_logits_kernel<FP8, 1 row>",
            "kernel_avg_us": d["kern_avg_ms"] * 1e3,
            "kernel_min_us_bracketed": d["kern_min_ms"] * 1e3,
            "algorithmic_bytes_per_launch": d["launch_bytes"],
        },
        "cpu_baseline": cpu,
    }
    if pre:
        line["prefill"] = {
            "workload": "chunked prefill: 16384 rows over 4096 keys, causal (r+1)//4, "
                        "budget 256e6 B (2 chunks), top-2048",
            "ms_per_call": pre["ms_per_call"],
            "tokens_per_s": pre["pairs"] / (pre["ms_per_call"] * 1e-3),
            "rows_scored": pre["rows_scored"],
            "fp8_flops_needed": pre["flops_needed"],
            "fp8_flops_all_rows": pre["flops"],
            "fp8_tflops_whole_call": pre["tflops_whole_call"],
            "fp8_mfma_frac_whole_call": pre["tflops_whole_call"] / FP8_MFMA_PEAK_TFLOPS,
            "note": "rows seeing at most k keys select all of them and are not scored; "
                    "the flops are those of the scored rows",
        }
        try:
            with open(MFMA_SUMMARY + ".json") as fh:
                mf = json.load(fh)
            if mf.get("kernel_source_digest") == prefill_source_digest():
                line["prefill"]["scoring_kernel_counters"] = {
                    "fp8_tflops": mf["fp8_tflops"], "fp8_mfma_frac": mf["fp8_mfma_frac"],
                    "us_per_dispatch": mf["us_per_dispatch"],
                    "source": "profiles/prefill_logits_fp8_chunked_mfma_counters.md"}
        except (OSError, ValueError, KeyError):
            pass
    if alt:
        line["decode_with_schedule_buffer"] = {
            "ms_per_step": alt["step_ms"], "ms_per_step_graph": alt["step_graph_ms"],
            "scoring_kernel_us": alt["kern_avg_ms"] * 1e3,
            "tokens_per_s": alt["tokens"] / (alt["step_ms"] * 1e-3)}
    if kvw:
        line["kv_cache_write"] = kvw
    if qq:
        line["query_quantization"] = qq
    if mla:
        line["sparse_attention"] = mla
    if others:
        line["other_decode_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
