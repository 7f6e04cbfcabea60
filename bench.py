"""Benchmark of one GVA decode step on one MI355X.

A step is the whole hot path over one batch: append each sequence's new token
(values + rotated positional key), absorb the per-head maps into the queries,
and run split-context decode attention with its merge.  The default workload
is the 350M-shaped decode: B=32, H=16, G=4, d_h=64, d_n=48, d_r=16, T=4096,
bf16 caches.  Inputs are synthetic and resident in HBM before timing starts;
the caches are cycled over enough copies (>= 1 GiB in total) that no step
finds its cache in the 256 MB last-level cache.

Prints ONE JSON line.  `value` is cache bytes read per second over whole
steps; `roofline` covers the decode kernel alone (HIP events around each of
its launches); `cpu_baseline` is the float64 oracle timed on host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py --decode-only --steps K   (decode launches alone, for
                                                  rocprofv3 --pmc runs)
       python bench.py --copy-calibration        (plain copy for counter scaling)
       python bench.py --ingest-counters FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
           (reads the four rocprofv3 --pmc output folders, writes
            profiles/traffic.json and profiles/<workload>_decode_traffic.txt)
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode-attn cache GB/s (% of HBM peak) and queries*ctx/s, "
          "350M shape, T=4096")
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
ROTATE_BYTES = 1 << 30

# Every timed leg times at least this many launches, whatever --steps is: a
# few graph replays alone read high (measured: 58.8 against 50.8 us per
# decode at the wide-rope shape with 3 replays against 25).
MIN_TIMED_LAUNCHES = 128


# Untimed replays before each timed region, for about this long: the GPU's
# clocks settle only after a spell of load (a decode timed right after a
# 20-step run read 54.7-58.8 us against 50.8 us after a 200-step run, at the
# wide-rope shape).
WARM_SECONDS = 0.1


def warm(torch, replay, seconds=WARM_SECONDS):
    """Replays `replay` (untimed) until `seconds` of wall time have passed,
    then queues one more without waiting: the caller's start event then
    lands behind work the GPU is still doing, so the host's submission of
    the first timed replay does not leave the GPU idle inside the timed
    region."""
    t = time.perf_counter()
    while True:
        for _ in range(4):
            replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t >= seconds:
            break
    replay()


def replays(steps, per_replay, at_least=1):
    """Graph replays to time: enough for `steps` launches and for
    MIN_TIMED_LAUNCHES, and at least `at_least`."""
    return max(at_least, -(-steps // per_replay), -(-MIN_TIMED_LAUNCHES // per_replay))

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["compressed_kv_cache_amd/csrc/gva_decode_mfma.hip",
                  "compressed_kv_cache_amd/csrc/gva_decode_ref.hip",
                  "compressed_kv_cache_amd/csrc/gva_device.h"]


def kernel_source_hash():
    """Hash of the decode kernels' code (comments and whitespace ignored), so
    counter-derived traffic is reported only for the code it was taken on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_350m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gqa", action="store_true")
    ap.add_argument("--no-multi", action="store_true",
                    help="skip the 4-query-token decode measurement")
    ap.add_argument("--no-rope-keys", action="store_true",
                    help="skip the rotated-reconstructed-key decode measurement")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill leg (every query token of the context at once)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the plain-read rate of the same cache buffers")
    ap.add_argument("--no-dr-sweep", action="store_true",
                    help="skip the decode timed over positional widths d_r = 0, 16, 24, 32")
    ap.add_argument("--no-vector-scores", action="store_true",
                    help="skip the decode timed with its scores on the vector units")
    ap.add_argument("--no-host-planned", action="store_true",
                    help="skip the decode timed with its split planned from host lengths")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long ragged workload's decode (both splits) beside "
                         "the 350M-shaped one")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--ingest-counters", nargs=4, metavar="DIR")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle sample")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration(torch, steps):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    n = COPY_BYTES
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "launches": steps}))


def counter_per_dispatch(folder, counter):
    """{kernel name: (average counter value per dispatch, dispatches)} from a
    rocprofv3 --pmc output folder (rows of one dispatch are summed)."""
    sums, disp = {}, {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"]
                sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: (sums[k] / len(disp[k]), len(disp[k])) for k in sums}


def pick_kernel(table, needle):
    hits = [(k, v) for k, v in table.items() if needle in k]
    if not hits:
        raise SystemExit(f"no kernel matching {needle!r} in counter output")
    return max(hits, key=lambda kv: kv[1][1])


def ingest_counters(dirs, workload):
    """HBM traffic of the decode kernel from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    known size."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    n_copy = COPY_BYTES
    _, (c_fetch, _) = pick_kernel(counter_per_dispatch(cfetch_dir, "FETCH_SIZE"), "copyBuffer")
    _, (c_write, _) = pick_kernel(counter_per_dispatch(cwrite_dir, "WRITE_SIZE"), "copyBuffer")
    name, (d_fetch, nd) = pick_kernel(counter_per_dispatch(fetch_dir, "FETCH_SIZE"),
                                      "decode_mfma_kernel")
    _, (d_write, _) = pick_kernel(counter_per_dispatch(write_dir, "WRITE_SIZE"),
                                  "decode_mfma_kernel")
    f_read = n_copy / 1024.0 / c_fetch
    f_write = n_copy / 1024.0 / c_write
    read_b = d_fetch * 1024.0 * f_read
    write_b = d_write * 1024.0 * f_write
    rec = {
        "kernel_source_hash": kernel_source_hash(),
        "kernel": name[:name.index(">(") + 1] if ">(" in name else name,
        "bytes_per_launch": round(read_b + write_b),
        "read_bytes_per_launch": round(read_b),
        "write_bytes_per_launch": round(write_b),
        "fetch_size_kib_per_dispatch": d_fetch,
        "write_size_kib_per_dispatch": d_write,
        "dispatches": nd,
        "copy_bytes": n_copy,
        "copy_fetch_size_kib": c_fetch,
        "copy_write_size_kib": c_write,
        "scale_read": f_read,
        "scale_write": f_write,
    }
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    table[workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps(rec))
    return rec


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch, max(1, args.steps))
        return
    import compressed_kv_cache_amd as gva
    import synthetic as syn

    dev = torch.device("cuda:0")
    cfg0 = syn.get_config(args.workload)
    cfg = syn.with_overrides(cfg0, append=True)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    x = syn.make_gva_inputs(cfg, device=dev)
    lens = x["seq_lens_host"]
    tokens = int(lens.sum())
    esize = 2 if cfg.cache_dtype == "bfloat16" else 4
    bytes_per_token = (cfg.G * cfg.d_h + cfg.d_r) * esize
    cache_bytes = tokens * bytes_per_token
    pool_bytes = (x["v_pool"].numel() + x["k_pool"].numel()) * esize
    R = max(1, math.ceil(ROTATE_BYTES / pool_bytes))
    pools = [(x["v_pool"], x["k_pool"])]
    for _ in range(R - 1):
        pools.append((x["v_pool"].clone(), x["k_pool"].clone()))
    ws = torch.zeros(gva.decode_workspace_bytes(cfg.B, cfg.H, x["v_pool"], x["k_pool"],
                                                x["block_table"], x["max_seq_len"]),
                     dtype=torch.uint8, device=dev)
    ws_step = torch.zeros(gva.decode_step_workspace_bytes(x["q_nope"], x["q_rope"], x["v_pool"],
                                                          x["k_pool"], x["block_table"],
                                                          x["max_seq_len"]),
                          dtype=torch.uint8, device=dev)
    qa = torch.empty((cfg.B, cfg.H, cfg.d_h + cfg.d_r), dtype=torch.float32, device=dev)
    out = torch.empty((cfg.B, cfg.H, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device=dev)

    def step(i):
        # append + absorb + decode: gva_decode_step, two launches
        vp, kp = pools[i % R]
        gva.decode_step(x["q_nope"], x["q_rope"], x["M"], vp, kp, x["block_table"],
                        x["seq_lens"], x["max_seq_len"], v_new=x["v_new"], k_new=x["k_new"],
                        rope_base=cfg.rope_base, workspace=ws_step, out=out, lse=lse)

    gva.absorb_query(x["q_nope"], x["q_rope"], x["M"], x["pos"], rope_base=cfg.rope_base,
                     out=qa)

    def decode_only(i):
        vp, kp = pools[i % R]
        gva.decode_attention(qa, vp, kp, x["block_table"], x["seq_lens"],
                             x["max_seq_len"], workspace=ws, out=out, lse=lse)

    if args.decode_only:  # decode launches alone, eager, over the rotating copies
        for i in range(args.warmup + args.steps):
            decode_only(i)
        torch.cuda.synchronize()
        print(json.dumps({"decode_only": cfg.name, "launches": args.warmup + args.steps,
                          "algorithmic_bytes_per_launch": cache_bytes}))
        return

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # eager: steps issued one by one from Python (launch overhead included)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / args.steps
    eager_out = out.clone()

    S = max(R, 8)
    # HIP graphs of S >= R consecutive steps (cycling over the rotating cache
    # copies; at least 8 so graph launch costs stay small), and of S decode
    # launches alone; replayed back to back.
    g_step, g_dec = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(S):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g_step):
        for i in range(S):
            step(i)
    # the timed region holds exactly `steps` steps: steps // S replays of the
    # S-step graph and one replay of a graph of the remaining steps
    full, rem = divmod(args.steps, S)
    g_rem = None
    if rem:
        g_rem = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rem):
            for i in range(rem):
                step(i)
    with torch.cuda.graph(g_dec):
        for i in range(S):
            decode_only(i)
    torch.cuda.synchronize()
    g_step.replay()
    torch.cuda.synchronize()
    graph_matches_eager = bool(torch.equal(out, eager_out))
    reps = replays(args.steps, S)
    if g_rem is not None:
        g_rem.replay()
    warm(torch, g_step.replay)
    t0.record()
    for _ in range(full):
        g_step.replay()
    if g_rem is not None:
        g_rem.replay()
    t1.record()
    torch.cuda.synchronize()
    steps_timed = full * S + rem
    ms_per_step = t0.elapsed_time(t1) / steps_timed

    # decode launches alone: one event pair per graph of S launches
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    warm(torch, g_dec.replay)
    for i in range(reps):
        evs[i][0].record()
        g_dec.replay()
        evs[i][1].record()
    torch.cuda.synchronize()
    dec_ms = sorted(a.elapsed_time(b) / S for a, b in evs)
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    dec_med_ms = dec_ms[len(dec_ms) // 2]
    print(f"[bench] step {ms_per_step * 1e3:.2f} us (eager {eager_ms * 1e3:.2f} us), "
          f"decode avg {dec_avg_ms * 1e3:.2f} us, graph==eager {graph_matches_eager}",
          file=sys.stderr, flush=True)

    value = cache_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = cache_bytes / (dec_avg_ms * 1e-3) / 1e9

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        rec = tr.get(cfg.name)
        if rec and rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("bytes_per_launch")
    except (OSError, ValueError):
        pass

    extra = {
        "queries_ctx_per_s": tokens / (ms_per_step * 1e-3),
        "head_queries_ctx_per_s": cfg.H * tokens / (ms_per_step * 1e-3),
        "pct_of_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
        "eager_ms_per_step": eager_ms,
        "graph_replay_matches_eager": graph_matches_eager,
        "decode_us_avg": dec_avg_ms * 1e3,
        "decode_us_median": dec_med_ms * 1e3,
        "decode_GBps": achieved,
        "cache_bytes_per_step": cache_bytes,
        "gqa_cache_bytes_same_shape": tokens * 2 * cfg.G * cfg.d_h * esize,
    }

    # the step's parts on their own (absorb: K1, append: K2, decode with its
    # merge: K3 + K4), each timed as graphs of back-to-back calls
    extra["per_call_us"] = {
        "absorb_query": time_calls(torch, lambda i: gva.absorb_query(
            x["q_nope"], x["q_rope"], x["M"], x["pos"], rope_base=cfg.rope_base, out=qa),
            args.steps),
        "append_cache": time_calls(torch, lambda i: gva.append_cache(
            x["v_new"], x["k_new"], x["pos"], x["block_table"], pools[i % R][0],
            pools[i % R][1], rope_base=cfg.rope_base), args.steps),
        "decode_attention": dec_avg_ms * 1e3,
        "decode_step": ms_per_step * 1e3,
    }

    if not args.no_read_probe:
        extra["read_probe"] = bench_read_probe(torch, gva, [vp for vp, _ in pools], dev,
                                               args.steps)
        extra["read_probe"]["decode_over_probe_rate"] = (
            achieved / extra["read_probe"]["cache_v_pool"]["GBps"])

    if not args.no_gqa and cfg.cache_dtype == "bfloat16":
        extra["gqa"] = bench_gqa(torch, gva, syn, cfg0, dev, args.steps, args.warmup)
        extra["gqa"]["time_ratio_gva_over_gqa"] = dec_avg_ms * 1e3 / extra["gqa"]["us_avg"]
        extra["gqa"]["byte_ratio_gva_over_gqa"] = (
            cache_bytes / extra["gqa_cache_bytes_same_shape"])
    if not args.no_dr_sweep and cfg.cache_dtype == "bfloat16" and cfg.name == "decode_350m":
        del pools
        torch.cuda.empty_cache()
        pools = None
        extra["dr_sweep"] = bench_dr_sweep(torch, gva, syn, cfg0, dev, args.steps,
                                           extra.get("gqa", {}).get("us_avg"))
    if not args.no_vector_scores and cfg.cache_dtype == "bfloat16" and cfg.H == 4 * cfg.G:
        extra["vector_scores"] = bench_vector_scores(torch, gva, syn, cfg0, dev, args.steps)
    # the split planned from host lengths: on ragged workloads only (on equal
    # lengths the plan is the max_seq_len split)
    if (not args.no_host_planned and cfg.cache_dtype == "bfloat16" and cfg.H == 4 * cfg.G
            and cfg.B <= 256 and cfg.T is None):
        extra["host_planned_split"] = bench_host_planned(torch, gva, syn, cfg0, dev, args.steps)
    if not args.no_long_context and cfg.name == "decode_350m":
        # the long-context workload (8 sequences of 1024 .. 131072 tokens,
        # shuffled blocks) at the 350M head shape, with its split planned
        # from the host lengths (its own kernel instance, so every launch of
        # the headline instance in this run is at the headline shape; the
        # max_seq_len split of this workload: --workload long_ragged)
        if pools is not None:
            del pools
            torch.cuda.empty_cache()
            pools = None
        lc = syn.get_config("long_ragged")
        extra["long_context"] = {"workload": lc.name,
                                 **bench_host_planned(torch, gva, syn, lc, dev, args.steps,
                                                      with_max_len=False)}
    if not args.no_multi:
        del pools
        torch.cuda.empty_cache()
        try:
            extra["multi_query"] = bench_multi(torch, gva, syn, cfg0, dev, args.steps,
                                               args.warmup, 4)
            extra["multi_query"]["time_ratio_over_one_query"] = (
                extra["multi_query"]["us_avg"] / (dec_avg_ms * 1e3))
        except gva.GvaError as e:  # widths with no multi-query kernel
            extra["multi_query"] = {"q_len": 4, "unsupported": str(e)}
    if not args.no_rope_keys and cfg.cache_dtype == "bfloat16":
        try:
            extra["rope_on_keys"] = bench_rope_keys(torch, gva, syn, cfg0, dev, args.steps)
        except gva.GvaError as e:
            extra["rope_on_keys"] = {"unsupported": str(e)}

    if not args.no_prefill and cfg.cache_dtype == "bfloat16" and cfg.T and cfg.T <= 8192:
        try:
            extra["prefill"] = bench_prefill(torch, gva, syn, cfg0, dev)
        except gva.GvaError as e:
            extra["prefill"] = {"unsupported": str(e)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg0, x, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.cache_dtype == "bfloat16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "B": cfg.B, "H": cfg.H, "G": cfg.G, "d_h": cfg.d_h,
            "d_n": cfg.d_n, "d_r": cfg.d_r,
            "T": cfg.T if cfg.T else "ragged",
            "context_tokens": tokens, "cache_dtype": cfg.cache_dtype,
            "accumulate": "f32",
            "step": "gva_decode_step: append+absorb (1 launch) + decode with in-kernel merge "
                    "(1 launch)",
            "timing": "HIP graphs of max(R, 8) steps replayed back to back, plus one graph "
                      "of the remaining steps: exactly --steps steps timed",
            "rotating_cache_copies": R,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "gva_decode_attention",
            "algorithmic_bytes_per_launch": cache_bytes,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


def bench_read_probe(torch, gva, v_pools, dev, steps):
    """Achievable read rate beside the 8 TB/s peak: the plain streaming read
    (gva_stream_read_probe: the decode's 16-byte non-temporal loads, no
    arithmetic) of (a) each rotating copy's value pool, the bulk of the
    cache bytes, one launch per copy like one decode launch, and (b) one
    1 GiB buffer in one launch, where the launch's fixed costs vanish.
    HIP events on the launch stream around graph replays."""
    out = torch.empty(gva.PROBE_BLOCKS, dtype=torch.int32, device=dev)

    def rate(bufs, launches):
        g = torch.cuda.CUDAGraph()
        for b in bufs:
            gva.stream_read_probe(b, out=out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(launches):
                gva.stream_read_probe(bufs[i % len(bufs)], out=out)
        warm(torch, g.replay)
        reps = replays(steps, launches)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (reps * launches) * 1e3
        nbytes = bufs[0].numel() * bufs[0].element_size()
        return {"bytes": nbytes, "us_avg": us, "GBps": nbytes / (us * 1e-6) / 1e9,
                "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}

    res = {"kernel": "gva_stream_read_probe",
           "cache_v_pool": rate(v_pools, max(len(v_pools), 8))}
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    res["one_gib"] = rate([big], 4)
    del big
    torch.cuda.empty_cache()
    return res


def time_calls(torch, call, steps, S=16):
    """Average time (us) of call(i): graphs of S calls replayed back to back,
    HIP events on the launch stream."""
    for i in range(S):
        call(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            call(i)
    warm(torch, g.replay)
    reps = replays(steps, S, 2)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * S) * 1e3


def time_decode(torch, gva, c, y, dev, steps, lens_host=None):
    """Average decode time (us) at config c with inputs y: graphs over
    rotating cache copies (at least 1 GiB, so no launch reads from L2 or
    the last-level cache what an earlier one left there), HIP events on the
    launch stream.  lens_host: time gva_decode_attention_lens (the split
    planned from these host lengths) instead."""
    pool_bytes = (y["v_pool"].numel() + y["k_pool"].numel()) * y["v_pool"].element_size()
    R = max(1, math.ceil(ROTATE_BYTES / pool_bytes))
    pools = [(y["v_pool"], y["k_pool"])] + [
        (y["v_pool"].clone(), y["k_pool"].clone()) for _ in range(R - 1)]
    qa = gva.absorb_query(y["q_nope"], y["q_rope"], y["M"], y["pos"], rope_base=c.rope_base)
    if lens_host is None:
        wsb = gva.decode_workspace_bytes(c.B, c.H, y["v_pool"], y["k_pool"], y["block_table"],
                                         y["max_seq_len"])
    else:
        wsb = gva.decode_workspace_bytes_lens(c.B, c.H, y["v_pool"], y["k_pool"],
                                              y["block_table"])
    ws = torch.zeros(max(16, wsb), dtype=torch.uint8, device=dev)
    out = torch.empty((c.B, c.H, c.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((c.B, c.H), dtype=torch.float32, device=dev)

    def launch(i):
        vp, kp = pools[i % R]
        if lens_host is None:
            gva.decode_attention(qa, vp, kp, y["block_table"], y["seq_lens"],
                                 y["max_seq_len"], workspace=ws, out=out, lse=lse)
        else:
            gva.decode_attention_lens(qa, vp, kp, y["block_table"], y["seq_lens"], lens_host,
                                      y["max_seq_len"], workspace=ws, out=out, lse=lse)

    S = max(R, 8)
    for i in range(S):
        launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            launch(i)
    warm(torch, g.replay)
    reps = replays(steps, S, 2)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / (reps * S) * 1e3
    del pools, g, qa, ws
    torch.cuda.empty_cache()
    return us


def bench_dr_sweep(torch, gva, syn, cfg, dev, steps, gqa_us):
    """The decode at one shape over positional widths d_r (d_n = d_h - d_r),
    same protocol as the headline decode (graphs over rotating cache copies,
    HIP events on the launch stream).  Beside each: the cache bytes, the
    fraction of the 8 TB/s peak, the closed-form GVA/GQA byte ratio
    1/2 + d_r/(2 G d_h) and the time ratio against the same-shape GQA decode
    (which does not depend on d_r)."""
    rows = []
    for d_r in (0, 16, 24, 32):
        c = syn.with_overrides(cfg, d_r=d_r, d_n=cfg.d_h - d_r)
        y = syn.make_gva_inputs(c, device=dev)
        tokens = int(y["seq_lens_host"].sum())
        byts = tokens * (c.G * c.d_h + c.d_r) * 2
        us = time_decode(torch, gva, c, y, dev, steps)
        row = {"d_r": d_r, "d_n": c.d_n, "us_avg": us, "cache_bytes": byts,
               "GBps": byts / (us * 1e-6) / 1e9,
               "frac_of_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
               "byte_ratio_gva_over_gqa": 0.5 + d_r / (2.0 * c.G * c.d_h)}
        if gqa_us:
            row["time_ratio_gva_over_gqa"] = us / gqa_us
        rows.append(row)
        del y
        torch.cuda.empty_cache()
    return {"shape": f"B={cfg.B} H={cfg.H} G={cfg.G} d_h={cfg.d_h} T={cfg.T}",
            "gqa_us_avg_same_shape": gqa_us, "rows": rows}


def bench_host_planned(torch, gva, syn, cfg, dev, steps, with_max_len=True):
    """The decode with its split planned from the host copy of the lengths
    (gva_decode_attention_lens), beside the split sized from max_seq_len
    unless with_max_len is false, on the workload's own lengths, same
    protocol as the headline decode."""
    y = syn.make_gva_inputs(cfg, device=dev)
    host = y["seq_lens_host"]
    tokens = int(host.sum())
    byts = tokens * (cfg.G * cfg.d_h + cfg.d_r) * 2
    res = {"tokens": tokens, "max_len": int(host.max()), "cache_bytes": byts}
    splits = (("split_by_max_seq_len", None),) if with_max_len else ()
    for name, lens in splits + (("host_planned", host),):
        us = time_decode(torch, gva, cfg, y, dev, steps, lens)
        res[name] = {"us_avg": us, "GBps": byts / (us * 1e-6) / 1e9,
                     "frac_of_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    if with_max_len:
        res["time_ratio_planned_over_max_len"] = (res["host_planned"]["us_avg"] /
                                                  res["split_by_max_seq_len"]["us_avg"])
    del y
    torch.cuda.empty_cache()
    return res


def bench_vector_scores(torch, gva, syn, cfg, dev, steps):
    """The decode with its scores on the vector units (GVA_DECODE_VALU=1:
    v_dot2_f32_bf16 over the same bf16 high and low query parts, the same
    streaming, staging, P.V and merge) beside the matrix-core decode, at the
    workload's shape, same protocol as the headline decode."""
    y = syn.make_gva_inputs(cfg, device=dev)
    tokens = int(y["seq_lens_host"].sum())
    byts = tokens * (cfg.G * cfg.d_h + cfg.d_r) * 2
    res = {"shape": f"B={cfg.B} H={cfg.H} G={cfg.G} d_h={cfg.d_h} d_r={cfg.d_r} T={cfg.T}",
           "cache_bytes": byts}
    for name, flag in (("matrix_scores", None), ("vector_scores", "1")):
        if flag:
            os.environ["GVA_DECODE_VALU"] = flag
        try:
            us = time_decode(torch, gva, cfg, y, dev, steps)
        finally:
            os.environ.pop("GVA_DECODE_VALU", None)
        res[name] = {"us_avg": us, "GBps": byts / (us * 1e-6) / 1e9,
                     "frac_of_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    res["time_ratio_vector_over_matrix"] = (res["vector_scores"]["us_avg"] /
                                            res["matrix_scores"]["us_avg"])
    del y
    torch.cuda.empty_cache()
    return res


def bench_multi(torch, gva, syn, cfg, dev, steps, warmup, L):
    """Decode of L query tokens per sequence (causal, the last L positions)
    over the same caches, same rotation protocol: the cache is read once for
    all L queries."""
    y = syn.make_gva_multi_inputs(cfg, L, device=dev)
    esize = 2 if cfg.cache_dtype == "bfloat16" else 4
    tokens = int(y["seq_lens_host"].sum())
    byts = tokens * (cfg.G * cfg.d_h + cfg.d_r) * esize
    pool_bytes = (y["v_pool"].numel() + y["k_pool"].numel()) * esize
    R = max(1, math.ceil(ROTATE_BYTES / pool_bytes))
    pools = [(y["v_pool"], y["k_pool"])] + [
        (y["v_pool"].clone(), y["k_pool"].clone()) for _ in range(R - 1)]
    qa = gva.absorb_query_multi(y["q_nope"], y["q_rope"], y["M"], y["pos"],
                                rope_base=cfg.rope_base)
    ws = torch.zeros(max(16, gva.decode_workspace_bytes_multi(
        cfg.B, cfg.H, L, y["v_pool"], y["k_pool"], y["block_table"], y["max_seq_len"])),
        dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.B, cfg.H, L, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, L), dtype=torch.float32, device=dev)

    def launch(i):
        vp, kp = pools[i % R]
        gva.decode_attention_multi(qa, vp, kp, y["block_table"], y["seq_lens"],
                                   y["max_seq_len"], workspace=ws, out=out, lse=lse)

    S = max(R, 8)
    for i in range(max(warmup, S)):
        launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            launch(i)
    warm(torch, g.replay)
    reps = replays(steps, S)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    avg = t0.elapsed_time(t1) / (reps * S)
    del pools, y
    torch.cuda.empty_cache()
    return {"q_len": L, "us_avg": avg * 1e3, "cache_bytes": byts,
            "GBps": byts / (avg * 1e-3) / 1e9,
            "queries_ctx_per_s": L * tokens / (avg * 1e-3)}


def bench_prefill(torch, gva, syn, cfg, dev, calls=10):
    """Prefill: every position of each sequence is a query (L = T), causal,
    through the blocked kernel.  Algorithmic work per (query, visible key)
    pair is 2*(2*d_h + d_r) flops (score over d_h + d_r, P.V over d_h);
    timed with HIP events on the launch stream around back-to-back calls."""
    L = int(cfg.T)
    y = syn.make_gva_multi_inputs(cfg, L, device=dev)
    qa = gva.absorb_query_multi(y["q_nope"], y["q_rope"], y["M"], y["pos"],
                                rope_base=cfg.rope_base)
    out = torch.empty((cfg.B, cfg.H, L, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H, L), dtype=torch.float32, device=dev)

    def launch():
        gva.decode_attention_multi(qa, y["v_pool"], y["k_pool"], y["block_table"],
                                   y["seq_lens"], y["max_seq_len"], out=out, lse=lse)

    warm(torch, launch)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        launch()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / calls
    lens = [int(n) for n in y["seq_lens_host"].tolist()]
    pairs = sum(sum(n - L + i + 1 for i in range(L)) for n in lens) * cfg.H
    flops = 2.0 * pairs * (2 * cfg.d_h + cfg.d_r)
    tflops = flops / (ms * 1e-3) / 1e12
    del y, qa
    torch.cuda.empty_cache()
    # the same-shape GQA prefill (keys and values cached per group, the
    # comparison the pages draw for prefill), same protocol
    z = syn.make_gqa_multi_inputs(cfg, L, device=dev)

    def launch_gqa():
        gva.gqa_decode_attention_multi(z["q"], z["k_pool"], z["v_pool"], z["block_table"],
                                       z["seq_lens"], z["max_seq_len"], out=out, lse=lse)

    warm(torch, launch_gqa)
    t0.record()
    for _ in range(calls):
        launch_gqa()
    t1.record()
    torch.cuda.synchronize()
    gqa_ms = t0.elapsed_time(t1) / calls
    del z, out, lse
    torch.cuda.empty_cache()
    return {"q_len": L, "ms_avg": ms, "query_key_pairs": pairs,
            "algorithmic_flops": flops,
            "gqa_ms_avg_same_shape": gqa_ms, "time_ratio_gva_over_gqa": ms / gqa_ms,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "kernel": "prefill_kernel"}}


def bench_rope_keys(torch, gva, syn, cfg, dev, steps):
    """The variant with ordinary RoPE on the reconstructed key (no positional
    slice, keys of width d_k = d_h) against the absorbed decode of the same
    cache (d_r = 0, the same bytes): both timed with the same protocol."""
    c0 = syn.with_overrides(cfg, d_n=cfg.d_h, d_r=0)
    y = syn.make_gva_inputs(c0, device=dev)
    tokens = int(y["seq_lens_host"].sum())
    byts = tokens * c0.G * c0.d_h * 2
    R = max(1, math.ceil(ROTATE_BYTES / (y["v_pool"].numel() * 2)))
    pools = [y["v_pool"]] + [y["v_pool"].clone() for _ in range(R - 1)]
    kp = y["k_pool"]
    out = torch.empty((c0.B, c0.H, c0.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((c0.B, c0.H), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(16, gva.decode_workspace_bytes(c0.B, c0.H, y["v_pool"], kp,
                                                        y["block_table"], y["max_seq_len"])),
                     dtype=torch.uint8, device=dev)
    wsr = torch.empty(1 << 26, dtype=torch.uint8, device=dev)
    qa = gva.absorb_query(y["q_nope"], y["q_rope"], y["M"], y["pos"])

    def rope(i):
        gva.decode_rope_keys(y["q_nope"], y["M"], pools[i % R], y["block_table"],
                             y["seq_lens"], y["max_seq_len"], rope_base=c0.rope_base,
                             workspace=wsr, out=out, lse=lse)

    def absorbed(i):
        gva.decode_attention(qa, pools[i % R], kp, y["block_table"], y["seq_lens"],
                             y["max_seq_len"], workspace=ws, out=out, lse=lse)

    res = {}
    S = max(R, 8)
    reps = max(1, replays(steps, S) // 4)
    for name, fn in (("rope_on_keys", rope), ("absorbed", absorbed)):
        for i in range(S):
            fn(i)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(S):
                fn(i)
        warm(torch, gr.replay)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            gr.replay()
        t1.record()
        torch.cuda.synchronize()
        res[name] = t0.elapsed_time(t1) / (reps * S) * 1e3
        del gr
    flops = 2.0 * tokens * c0.H * c0.d_h * c0.d_n
    del pools, y
    torch.cuda.empty_cache()
    return {"d_k": c0.d_n, "cache_bytes": byts, "us_avg": res["rope_on_keys"],
            "absorbed_us_avg_same_cache": res["absorbed"],
            "time_ratio_over_absorbed": res["rope_on_keys"] / res["absorbed"],
            "key_rebuild_TFLOPs": flops / (res["rope_on_keys"] * 1e-6) / 1e12}


def bench_gqa(torch, gva, syn, cfg, dev, steps, warmup):
    """Same-shape GQA decode (key and value streams), same rotation protocol."""
    y = syn.make_gqa_inputs(cfg, device=dev)
    esize = 2
    tokens = int(y["seq_lens_host"].sum())
    byts = tokens * 2 * cfg.G * cfg.d_h * esize
    pool_bytes = 2 * y["v_pool"].numel() * esize
    R = max(1, math.ceil(ROTATE_BYTES / pool_bytes))
    pools = [(y["k_pool"], y["v_pool"])] + [
        (y["k_pool"].clone(), y["v_pool"].clone()) for _ in range(R - 1)]
    out = torch.empty((cfg.B, cfg.H, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.H), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(16, gva.gqa_decode_workspace_bytes(
        cfg.B, cfg.H, y["k_pool"], y["v_pool"], y["block_table"], y["max_seq_len"])),
        dtype=torch.uint8, device=dev)

    def launch(i):
        kp, vp = pools[i % R]
        gva.gqa_decode_attention(y["q"], kp, vp, y["block_table"], y["seq_lens"],
                                 y["max_seq_len"], workspace=ws, out=out, lse=lse)

    S = max(R, 8)
    for i in range(max(warmup, S)):
        launch(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            launch(i)
    warm(torch, g.replay)
    reps = replays(steps, S)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    avg = t0.elapsed_time(t1) / (reps * S)
    del pools, y
    torch.cuda.empty_cache()
    return {"us_avg": avg * 1e3, "cache_bytes": byts, "GBps": byts / (avg * 1e-3) / 1e9}


def cpu_model_name():
    """The host CPU's model name (the lscpu 'Model name' line, read from
    /proc/cpuinfo), or None where it cannot be read."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, x, target_s):
    """The float64 oracle on the host: whole sequences of the same workload,
    as many as fit the time target, scaled to cache GB/s."""
    import numpy as np
    import oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    h = {k: v.detach().cpu() for k, v in x.items() if hasattr(v, "detach")}
    esize = 2 if cfg.cache_dtype == "bfloat16" else 4
    per_tok = (cfg.G * cfg.d_h + cfg.d_r) * esize
    vp, kp = o.to_f64(h["v_pool"]), o.to_f64(h["k_pool"])
    done_tokens, spent, seqs = 0, 0.0, 0
    order = list(range(cfg.B))
    while spent < target_s:
        b = order[seqs % cfg.B]
        t = time.perf_counter()
        o.gva_decode_materialized(h["q_nope"], h["q_rope"], h["M"], vp, kp,
                                  h["block_table"], h["seq_lens"], base=cfg.rope_base,
                                  seqs=[b])
        spent += time.perf_counter() - t
        done_tokens += int(h["seq_lens_host"][b])
        seqs += 1
    gbs = done_tokens * per_tok / spent / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model_name(), "host_cpus": os.cpu_count(),
            "sample": f"{seqs} whole sequences ({done_tokens} context tokens x {cfg.H} heads)"
                      f" of {cfg.name}, float64, keys materialised, {spent:.1f} s",
            "queries_ctx_per_s": done_tokens / spent}


if __name__ == "__main__":
    main()
