#!/usr/bin/env python3
"""Decode-step throughput of the positions-aware cached decode path on one MI355X.

One step = one layer of the whole hot path on one batch of synthetic input:
RoPE(K) + K/V store into the shared slot cache, RoPE(Q), causal GQA attention
over every row's prefix with the keys of all rows shared evenly by the resident
waves, then the cross-wave merge to the BF16 output.
Steps rotate over several layer caches (as a multi-layer decode does), so a
step never finds its K/V bytes left in the 256 MB last-level cache by the
previous step: 4 layers of 1 GiB by default.  The warm-up reads every rotated
layer once: the first decode read of a freshly allocated layer measured about
25 us slower on MI355X than every later one.

Prints one JSON line: KV GB/s (algorithmic K+V prefix bytes per step / step
time), % of the 8 TB/s HBM peak, tokens/s, the dominant kernel's roofline
point (its own duration from HIP events the library records around it), and
the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, published
EVENT_STRIDE = 10         # timed decode steps per step whose kernel carries HIP events
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak, published
METRIC = "decode attn step: KV GB/s and % of HBM peak; tokens/s at A rows, ctx"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b", choices=["llama3_8b", "ragged", "long"])
    ap.add_argument("--layers", type=int, default=4,
                    help="layer caches rotated over the steps (at most the warm-up count, so "
                         "every layer is read once before the timed region)")
    ap.add_argument("--batch", type=int, default=0,
                    help="decode entries A in place of the workload's own (0 = as configured); "
                         "the workload is then named <workload>_decode_A<batch>")
    ap.add_argument("--waves", type=int, default=0,
                    help="waves sharing the keys (0 = the device's resident waves)")
    ap.add_argument("--kernel", type=int, default=0, help="0 tuned stream, 1 readable")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU-oracle sample (0 = skip)")
    ap.add_argument("--graph-reps", type=int, default=25,
                    help="replays of a graph of all layers' steps (0 = skip)")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="also time the equal-length batched prefill (0 = skip)")
    ap.add_argument("--chunk-steps", type=int, default=20,
                    help="also time the prefill chunk of mixed starts and lengths (0 = skip)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="storage type of the cache and tensors of the headline run")
    ap.add_argument("--sched-boundaries", type=int, default=2000,
                    help="also time the slot manager's step boundary (0 = skip)")
    ap.add_argument("--f16-steps", type=int, default=50,
                    help="also time the decode step and the prefill with FP16 storage (0 = skip)")
    ap.add_argument("--other-decode-steps", type=int, default=-1,
                    help="timed steps of the ragged and long-context decode legs (-1 = --steps, "
                         "0 = skip)")
    ap.add_argument("--other-layers", type=int, default=4,
                    help="layer caches rotated in the ragged and long-context legs")
    ap.add_argument("--ceiling-reps", type=int, default=5,
                    help="timed reads per launch shape of the streaming-read ceiling (0 = skip)")
    ap.add_argument("--fold-counters", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="fold two rocprofv3 --pmc counter_collection.csv files of one bench leg "
                         "(FETCH_SIZE, then WRITE_SIZE) into profiles/counters.json under the "
                         "workload's label, scaled by the copy reference, and exit")
    ap.add_argument("--fold-copy", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="fold the two counter runs of --copy-reference (the scale of "
                         "FETCH_SIZE and WRITE_SIZE) into profiles/counters.json, and exit")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase timeline of the decode stream kernel on --workload from "
                         "per-group wall-clock stamps (needs the stamps build: python -m "
                         "positions_aware_cached_amd.build --stamps); one JSON line")
    ap.add_argument("--trace-phases", metavar="KERNEL_TRACE_CSV",
                    help="stream kernel, merge kernel and the gaps between them, from a "
                         "rocprofv3 --kernel-trace CSV of a decode bench run; one JSON line")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device copy (5 times): the reference that "
                         "scales the HBM byte counters of a profiler run")
    return ap.parse_args()


def hip_runtime():
    """The HIP runtime torch loaded (one runtime per process)."""
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                L = ctypes.CDLL(line.split()[-1])
                L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
                L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
                L.hipEventDestroy.argtypes = [ctypes.c_void_p]
                L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
                return L
    raise RuntimeError("HIP runtime not loaded")


# HIP event flag: no system-scope fence (cache writeback and invalidation) when
# the event is recorded.  The bench's events only time kernels and are read
# after a device-wide synchronize, so the fence buys nothing and, on MI355X,
# delays the work queued after the event's kernel by several microseconds.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
TIMING_EVENT_FLAGS = HIP_EVENT_DISABLE_SYSTEM_FENCE


def timing_event(hip, h):
    """Create a timing event into the c_void_p h; returns the HIP status."""
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    return hip.hipEventCreateWithFlags(ctypes.byref(h), TIMING_EVENT_FLAGS)


def percentile(xs, q):
    """Linear-interpolation percentile (numpy's default rule)."""
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
CSRC = os.path.join(ROOT, "positions_aware_cached_amd", "csrc")
# the sources each kernel is built from: a counter summary stays valid for a
# kernel while their code (comments and whitespace aside) is unchanged
KERNEL_SOURCES = {"decode": ("decode.hip", "kernels.h", "elem.h"),
                  "prefill": ("prefill.hip", "kernels.h", "elem.h")}


def source_digest(family, csrc=CSRC):
    """Digest of one kernel family's sources ("decode" or "prefill"): sha256
    of the code with comments and whitespace removed, so an edit of the
    comments alone keeps the profiler figures taken on that code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def decode_label(args):
    """Name of the decode workload: the configuration, and the batch size when overridden."""
    return f"{args.workload}_decode" + (f"_A{args.batch}" if args.batch else "")


def decode_config(args, dtype):
    import workloads
    cfg = workloads.config(args.workload, dtype=dtype)
    if args.batch:
        cfg = workloads.config(args.workload, dtype=dtype, A=args.batch,
                               S=max(cfg["S"], args.batch))
    return cfg


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed profiler summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter on a plain copy of known size),
    or None when the summary is missing or was taken on other kernel sources."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    e = c.get("kernels", {}).get(f"{kernel}@{workload}")
    if e is None:
        return None
    family = "decode" if kernel.startswith("k_decode") else "prefill"
    if e.get("source_digest") != source_digest(family):
        return None
    return e.get("hbm_bytes_per_launch")


def _counter_means(path, counter):
    """Mean value per dispatch of `counter`, by short kernel name (k_* kernels and
    the runtime's copy kernel), from a rocprofv3 counter_collection.csv."""
    import csv
    import re
    sums, counts = {}, {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            m = re.search(r"\b(k_[a-z0-9_]+|__amd_rocclr_copyBuffer)\b", r["Kernel_Name"])
            if not m:
                continue
            k = m.group(1)
            sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
            counts[k] = counts.get(k, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def _load_counters():
    try:
        with open(COUNTERS) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {"kernels": {}}


def _save_counters(c):
    with open(COUNTERS, "w") as f:
        json.dump(c, f, indent=1, sort_keys=True)
        f.write("\n")


def fold_copy(fetch_csv, write_csv):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the 1 GiB device copy of
    --copy-reference: their ratio to the bytes copied scales every kernel's
    counters to bytes."""
    n = 1 << 30
    fk = _counter_means(fetch_csv, "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    wk = _counter_means(write_csv, "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    c = _load_counters()
    c["copy_reference"] = {"bytes": n, "fetch_kib": fk, "write_kib": wk,
                           "fetch_scale": n / (fk * 1024.0), "write_scale": n / (wk * 1024.0)}
    _save_counters(c)
    print(json.dumps(c["copy_reference"]))


def fold_counters(label, fetch_csv, write_csv):
    """HBM bytes per launch of the k_* kernels of one workload's bench leg:
    FETCH_SIZE and WRITE_SIZE means, each scaled by the copy reference, stored
    with the digest of the kernel family's sources (used only while it matches)."""
    c = _load_counters()
    ref = c.get("copy_reference")
    assert ref, "fold the copy reference first (--fold-copy)"
    family = "decode" if label.endswith("decode") or "_decode_" in label else "prefill"
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    for k in sorted(set(fetch) & set(write)):
        if not k.startswith("k_" + family):
            continue
        fb = fetch[k] * 1024.0 * ref["fetch_scale"]
        wb = write[k] * 1024.0 * ref["write_scale"]
        c["kernels"][f"{k}@{label}"] = {
            "source_digest": source_digest(family), "fetch_kib_raw": fetch[k],
            "write_kib_raw": write[k], "fetch_bytes": int(round(fb)), "write_bytes": int(round(wb)),
            "hbm_bytes_per_launch": int(round(fb + wb))}
        print(k, label, c["kernels"][f"{k}@{label}"])
    _save_counters(c)


def decode_phases(args, calls=24):
    """Timeline of the decode stream kernel, per launch, from the stamps build:
    each work group records the wall clock (100 MHz) at entry, when its plan is
    known, when its first tile has landed and at exit.  Times are in us from the
    earliest group entry of the launch; the kernel's own duration comes from HIP
    events around its dispatch.  Phases (medians over the launches):
      start     event duration minus (last exit - first entry): dispatch, first
                wave start and drain after the last wave;
      plan      median group time from entry to a known first tile;
      ramp      median (and max) first tile landed: all groups request their
                first tiles at once, so this is the time HBM takes to serve them;
      steady    from the median first tile to the 10th-percentile group exit;
      tail      10th-percentile to last group exit (groups finishing unevenly)."""
    import torch

    from positions_aware_cached_amd import build as pbuild
    import positions_aware_cached_amd as pac
    import workloads

    if not os.path.exists(pbuild.STAMPS_LIB):
        sys.exit("bench.py --phases needs the stamps build: "
                 "python -m positions_aware_cached_amd.build --stamps")
    L = pac.load(pbuild.STAMPS_LIB)
    L.mllm_debug_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    hip = hip_runtime()
    dev = torch.device("cuda:0")
    cfg = decode_config(args, "bf16")
    A, Hq, D = cfg["A"], cfg["Hq"], cfg["D"]
    inp = workloads.draw_decode(cfg, device="cuda")
    nl = max(1, args.layers)
    layers = [(inp["Kc"], inp["Vc"])] + workloads.draw_cache_layers(cfg, nl - 1)
    cache = pac.Cache.wrap([k for k, _ in layers], [v for _, v in layers])
    pos = torch.as_tensor(inp["positions"], device=dev)
    rows = torch.as_tensor(inp["rows"], device=dev)
    out = torch.empty((A, Hq, D), dtype=inp["q"].dtype, device=dev)
    mirror = np.concatenate([inp["positions"], inp["rows"]]).astype(np.int32)
    ws = torch.zeros(pac.decode_workspace_size(cache, A, Hq, int(inp["positions"].max())),
                     dtype=torch.uint8, device=dev)
    call = pac.DecodeCall(cache, inp["q"], inp["k_new"], inp["v_new"], pos, rows, out, ws,
                          cfg["base"], host_mirror=mirror)
    for i in range(max(args.warmup, nl)):
        call(i % nl)
    torch.cuda.synchronize()
    nslot = 4096 * 8
    rec = {k: [] for k in ("event", "start", "plan", "ramp_med", "ramp_max", "steady",
                           "tail", "exit_p10", "exit_med", "exit_max", "exit_first_half",
                           "exit_second_half", "exit_sd_first_half", "exit_sd_second_half")}
    groups = 0
    for i in range(calls):
        pair = (ctypes.c_void_p * 2)()
        for j in range(2):
            h = ctypes.c_void_p()
            assert timing_event(hip, h) == 0
            pair[j] = h.value
        st = np.zeros(nslot, dtype=np.uint64)
        call(i % nl, attn_events=pair)
        torch.cuda.synchronize()
        assert L.mllm_debug_stamps(st.ctypes.data, st.nbytes) == 0
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(pair[0]),
                                       ctypes.c_void_p(pair[1])) == 0
        for j in range(2):
            hip.hipEventDestroy(ctypes.c_void_p(pair[j]))
        g = st.reshape(4096, 8).astype(np.int64)
        # only the groups of this launch: entries before their exits, exits
        # after the launch's earliest entry (stale slots of larger launches)
        live = (g[:, 0] > 0) & (g[:, 3] >= g[:, 0])
        t0 = g[live, 0].min()
        live &= g[:, 3] >= t0
        idx = np.nonzero(live)[0]
        g = g[live]
        groups = len(g)
        # groups w < NS / 2 are each compute unit's first-dispatched group
        first = idx < (idx.max() + 1) // 2
        rel = (g - t0) * 0.01
        ev = f.value * 1e3
        ex = rel[:, 3]
        rec["event"].append(ev)
        rec["start"].append(ev - ex.max())
        rec["plan"].append(float(np.median(rel[:, 1])))
        rec["ramp_med"].append(float(np.median(rel[:, 7])))
        rec["ramp_max"].append(float(rel[:, 7].max()))
        rec["exit_p10"].append(float(np.percentile(ex, 10)))
        rec["exit_med"].append(float(np.median(ex)))
        rec["exit_max"].append(float(ex.max()))
        rec["exit_first_half"].append(float(np.mean(ex[first])))
        rec["exit_second_half"].append(float(np.mean(ex[~first])))
        rec["exit_sd_first_half"].append(float(np.std(ex[first])))
        rec["exit_sd_second_half"].append(float(np.std(ex[~first])))
        rec["steady"].append(rec["exit_p10"][-1] - rec["ramp_med"][-1])
        rec["tail"].append(rec["exit_max"][-1] - rec["exit_p10"][-1])
    res = {"workload": decode_label(args), "launches": calls, "groups": groups,
           "unit": "us", "source": "per-group wall-clock stamps (stamps build)"}
    for k, v in rec.items():
        res[k] = round(float(np.median(v)), 2)
    print(json.dumps(res))


def trace_phases(path):
    """From a rocprofv3 kernel trace of a decode bench run, over back-to-back
    steps (stream kernel, merge kernel, next stream kernel less than 50 us
    apart): the stream and merge kernels' durations, the share of steps whose
    kernels run with no gap between them (under 1 us), and the gaps of the
    other steps: those that carry timing events (every few steps of the timed
    loop; each event pair delays the work behind it) and the per-step
    distribution pass.  Medians in us."""
    import csv
    import re
    ks = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            m = re.search(r"\b(k_decode_[a-z_]+)\b", r["Kernel_Name"])
            if m:
                ks.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), m.group(1)))
    ks.sort()
    stream, merge, g1s, g2s, free = [], [], [], [], 0
    for i in range(len(ks) - 2):
        (s0, e0, n0), (s1, e1, n1), (s2, e2, n2) = ks[i], ks[i + 1], ks[i + 2]
        if n0 != "k_decode_stream" or not n1.startswith("k_decode_merge") or n2 != n0:
            continue
        g1, g2 = (s1 - e0) / 1e3, (s2 - e1) / 1e3
        if g1 > 50 or g2 > 50:
            continue
        stream.append((e0 - s0) / 1e3)
        merge.append((e1 - s1) / 1e3)
        if g1 < 1 and g2 < 1:
            free += 1
        else:
            g1s.append(g1)
            g2s.append(g2)
    med = lambda x: round(float(np.median(x)), 2) if x else None
    print(json.dumps({"unit": "us", "steps": len(stream), "stream": med(stream),
                      "merge": med(merge), "gap_free_steps": free,
                      "steps_with_gaps": len(g1s), "gap_to_merge": med(g1s),
                      "gap_to_next_step": med(g2s), "source": os.path.basename(path)}))


def copy_reference():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": n, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.fold_copy:
        fold_copy(*args.fold_copy)
        return
    if args.fold_counters:
        fold_counters(*args.fold_counters)
        return
    if args.copy_reference:
        copy_reference()
        return
    if args.trace_phases:
        trace_phases(args.trace_phases)
        return
    if args.phases:
        decode_phases(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path runs on one GPU, rows shard across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import positions_aware_cached_amd as pac
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = hip_runtime()
    d = decode_leg(args, hip, args.dtype, args.steps, args.warmup, args.layers)
    cfg, inp, cache, pos, rows, out, ws, mirror, call = (d[k] for k in (
        "cfg", "inp", "cache", "pos", "rows", "out", "ws", "mirror", "call"))
    A, S, C, Hq, Hkv, D = (cfg[k] for k in ("A", "S", "C", "Hq", "Hkv", "D"))
    pos_h, rows_h, ctx = d["pos_h"], d["rows_h"], d["ctx"]
    kv_bytes, total_bytes, wall, attn_ms, step_ms = (d[k] for k in (
        "kv_bytes", "total_bytes", "wall", "attn_ms", "step_ms"))
    K, W, L = args.steps, args.warmup, args.layers
    ms_per_step = wall * 1e3 / K
    kv_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    tot_gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    attn_avg = float(np.mean(attn_ms))
    attn_gbs = kv_bytes / (attn_avg * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": decode_label(args), "A": A, "slots": S, "capacity": C,
                   "h_q": Hq, "h_kv": Hkv, "head_dim": D, "rope_base": cfg["base"],
                   "ctx_mean": round(float(ctx.mean()), 1), "ctx_max": int(ctx.max()),
                   "layers_rotated": L, "waves": args.waves or "resident",
                   "kernel": "fused stream" if args.kernel == 0 else "readable"},
        "pct_hbm_peak": round(100.0 * tot_gbs / PEAK_HBM_GBS, 2),
        "total_gbs": round(tot_gbs, 1),
        "tokens_per_s": round(A / (ms_per_step * 1e-3), 1),
        "step_ms_median": round(percentile(step_ms, 50), 4),
        "step_ms_p95": round(percentile(step_ms, 95), 4),
        "kv_bytes_per_step": kv_bytes,
        "total_bytes_per_step": total_bytes,
        "roofline": {
            "kernel": "k_decode_stream" if args.kernel == 0 else "k_decode_readable",
            "bound": "hbm",
            "achieved": round(attn_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("k_decode_stream" if args.kernel == 0 else
                                        "k_decode_readable", decode_label(args)
                                        + ("_f16" if args.dtype == "f16" else "")),
            "avg_launch_ms": round(attn_avg, 5),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }

    if args.graph_reps > 0:
        res["graph"] = bench_graph(args, cache, inp, pos, rows, out, ws, mirror, cfg, kv_bytes)
    if args.prefill_steps > 0:
        res["prefill"] = bench_prefill(args, hip, "prefill", args.prefill_steps)
    if args.chunk_steps > 0:
        res["chunk"] = bench_prefill(args, hip, "chunk", args.chunk_steps)
    if args.f16_steps > 0 and args.dtype != "f16":
        res["f16"] = bench_f16(args, hip)
    if args.sched_boundaries > 0:
        res["sched"] = bench_sched(args, ms_per_step)
    if args.cpu_seconds > 0:
        call(0)  # a fresh layer-0 step: the oracle sample is compared with it
        torch.cuda.synchronize()
        res["cpu_baseline"] = cpu_baseline(args, cfg, inp, d["layers"], pos_h, rows_h, out)
    # the ragged and long-context decode batches, after the headline leg's memory is freed
    K2 = args.steps if args.other_decode_steps < 0 else args.other_decode_steps
    if K2 > 0 and args.workload == "llama3_8b" and not args.batch:
        del d, inp, cache, out, ws, call
        torch.cuda.empty_cache()
        for w in ("ragged", "long"):
            res[w] = bench_decode_workload(args, hip, w, K2)
            torch.cuda.empty_cache()
    if args.ceiling_reps > 0:
        ceil = read_ceiling(args.ceiling_reps)
        res["ceiling"] = ceil
        for leg in [res] + [res[w] for w in ("ragged", "long") if w in res]:
            leg["roofline"]["ceiling_gbs"] = ceil["ceiling_gbs"]
            leg["roofline"]["frac_of_ceiling"] = round(
                leg["roofline"]["achieved"] / ceil["ceiling_gbs"], 4)
    print(json.dumps(res), flush=True)


def decode_leg(args, hip, dtype, K, W, L):
    """The decode step on the --workload configuration with storage type dtype:
    W warm-up and K timed steps rotating over L layer caches; the attention
    kernel's own duration from events stamped in its dispatch."""
    import torch

    import positions_aware_cached_amd as pac
    import workloads

    dev = torch.device("cuda:0")
    cfg = decode_config(args, dtype)
    A, S, C, Hq, Hkv, D = (cfg[k] for k in ("A", "S", "C", "Hq", "Hkv", "D"))
    print(f"[bench] drawing {args.workload} {dtype} inputs + {L} layer caches", file=sys.stderr,
          flush=True)
    inp = workloads.draw_decode(cfg, device="cuda")
    layers = [(inp["Kc"], inp["Vc"])] + workloads.draw_cache_layers(cfg, L - 1)
    cache = pac.Cache.wrap([k for k, _ in layers], [v for _, v in layers])
    pos_h, rows_h = inp["positions"], inp["rows"]
    pos = torch.as_tensor(pos_h, device=dev)
    rows = torch.as_tensor(rows_h, device=dev)
    out = torch.empty((A, Hq, D), dtype=inp["q"].dtype, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    mirror = np.concatenate([pos_h, rows_h]).astype(np.int32)
    nws = pac.decode_workspace_size(cache, A, Hq, int(pos_h.max()), args.waves,
                                    args.kernel)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    call = pac.DecodeCall(cache, inp["q"], inp["k_new"], inp["v_new"], pos, rows, out, ws,
                          cfg["base"], host_mirror=mirror, status=status,
                          waves=args.waves, kernel=args.kernel)

    # algorithmic bytes of one step
    ctx = pos_h.astype(np.int64) + 1
    kv_bytes = int(ctx.sum()) * Hkv * D * 2 * 2
    io_bytes = A * Hq * D * 2 * 2 + 2 * A * Hkv * D * 2 * 2 + 8 * A
    total_bytes = kv_bytes + io_bytes

    # The attention kernel's own duration: the library stamps start and end
    # events into the dispatch of every EVENT_STRIDE-th timed step (2 of the
    # 20 timed steps of a short run, 20 of 200).  A stamped dispatch delays
    # its step by about 9 us on MI355X (kernel trace: 4.5 us before the kernel,
    # 4.5 us before the merge), so the other steps run unstamped.
    stamped = [i for i in range(K) if i % EVENT_STRIDE == EVENT_STRIDE - 1] or [K - 1]
    evs = {}
    for i in stamped:
        pair = (ctypes.c_void_p * 2)()
        for j in range(2):
            h = ctypes.c_void_p()
            assert timing_event(hip, h) == 0
            pair[j] = h.value
        evs[i] = pair

    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for i in range(W):
        call(i % L)
    torch.cuda.synchronize()
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call(i % L, attn_events=evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(status.item()) == 0, "device reported an index error"
    attn_ms = []
    for pair in evs.values():
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(pair[0]),
                                       ctypes.c_void_p(pair[1])) == 0
        attn_ms.append(f.value)
        hip.hipEventDestroy(ctypes.c_void_p(pair[0]))
        hip.hipEventDestroy(ctypes.c_void_p(pair[1]))
    # per-step distribution from a separate untimed pass (events between steps
    # add queue commands, so they stay out of the timed region)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(min(K, 100))]
    for i, (e0, e1) in enumerate(step_ev):
        e0.record()
        call(i % L)
        e1.record()
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in step_ev]

    return dict(cfg=cfg, inp=inp, cache=cache, pos=pos, rows=rows, out=out, ws=ws, mirror=mirror,
                call=call, status=status, layers=layers, pos_h=pos_h, rows_h=rows_h, ctx=ctx, kv_bytes=kv_bytes,
                total_bytes=total_bytes, wall=wall, attn_ms=attn_ms, step_ms=step_ms)


def bench_decode_workload(args, hip, workload, K):
    """The decode step on another batch shape ("ragged": 200 rows of 256 with
    log-uniform positions; "long": 8 rows of 32K context, 64 query heads): K
    timed steps after the headline's warm-up count, rotating over
    --other-layers layer caches; figures as in the headline line."""
    import argparse
    a = argparse.Namespace(**vars(args))
    a.workload, a.batch = workload, 0
    L = max(1, args.other_layers)
    d = decode_leg(a, hip, "bf16", K, args.warmup, L)
    cfg, ctx, kv = d["cfg"], d["ctx"], d["kv_bytes"]
    ms = d["wall"] * 1e3 / K
    attn = float(np.mean(d["attn_ms"]))
    gbs = kv / (ms * 1e-3) / 1e9
    agbs = kv / (attn * 1e-3) / 1e9
    label = decode_label(a)
    res = {"workload": label, "A": cfg["A"], "slots": cfg["S"], "capacity": cfg["C"],
           "h_q": cfg["Hq"], "h_kv": cfg["Hkv"], "head_dim": cfg["D"],
           "ctx_mean": round(float(ctx.mean()), 1), "ctx_max": int(ctx.max()),
           "layers_rotated": L, "steps": K, "ms_per_step": round(ms, 4),
           "value": round(gbs, 1), "unit": "GB/s",
           "pct_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
           "tokens_per_s": round(cfg["A"] / (ms * 1e-3), 1),
           "step_ms_median": round(percentile(d["step_ms"], 50), 4),
           "kv_bytes_per_step": kv,
           "roofline": {"kernel": "k_decode_stream", "bound": "hbm", "achieved": round(agbs, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(agbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic("k_decode_stream", label),
                        "avg_launch_ms": round(attn, 5), "algorithmic_bytes_per_launch": kv}}
    del d
    return res


def read_ceiling(reps):
    """Streaming-read ceiling of the device: a plain non-temporal read of 4 GiB
    (positions_aware_cached_amd/probe/read_ceiling.hip), timed over `reps`
    reads per launch shape; the best median over three shapes (blocks of 256
    lanes per compute unit x loads in flight per lane)."""
    import torch
    path = os.path.join(ROOT, "positions_aware_cached_amd", "libreadprobe.so")
    L = ctypes.CDLL(path)
    L.mllm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    n = 4 << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 4 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for bpc, unroll in ((3, 2), (2, 4), (1, 8)):
        ms = []
        for r in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = L.mllm_probe_read(buf.data_ptr(), n, cus * bpc, unroll, sink.data_ptr(), stream)
            e1.record()
            assert rc == 0, f"read probe launch failed ({rc})"
            torch.cuda.synchronize()
            if r:
                ms.append(e0.elapsed_time(e1))
        med = float(np.median(ms))
        gbs = n / (med * 1e-3) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, bpc, unroll, med)
    del buf, sink
    torch.cuda.empty_cache()
    return {"ceiling_gbs": round(best[0], 1), "frac_of_peak": round(best[0] / PEAK_HBM_GBS, 4),
            "bytes": n, "ms": round(best[3], 4),
            "launch": f"{best[1]} blocks of 256 lanes per CU, {best[2]} 16-B loads in flight per "
                      "lane, non-temporal", "reads_per_shape": reps}


def bench_f16(args, hip):
    """The decode step and the 16 x 1024 prefill with FP16 storage (same
    kernels, FP16 operands): the same figures as the BF16 lines."""
    K = args.f16_steps
    d = decode_leg(args, hip, "f16", K, min(args.warmup, K), args.layers)
    ms = d["wall"] * 1e3 / K
    attn = float(np.mean(d["attn_ms"]))
    kv = d["kv_bytes"]
    res = {"decode": {"workload": decode_label(args), "steps": K,
                      "ms_per_step": round(ms, 4), "value": round(kv / (ms * 1e-3) / 1e9, 1),
                      "unit": "GB/s",
                      "roofline": {"kernel": "k_decode_stream", "bound": "hbm",
                                   "achieved": round(kv / (attn * 1e-3) / 1e9, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(kv / (attn * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "avg_launch_ms": round(attn, 5)}}}
    del d
    if args.prefill_steps > 0:
        res["prefill"] = bench_prefill(args, hip, "prefill", args.prefill_steps, dtype="f16")
    return res


def bench_sched(args, step_ms):
    """Host cost of the slot manager's step boundary in steady serving: 64 rows
    (the decode batch of the headline workload), requests of 128-512 prompt and
    64-256 new tokens arriving so that the queue never empties; row lengths are
    advanced as the prefill and decode calls would.  Timed: the boundary calls
    only: `boundary_us` is the library call through ctypes (the plan left in
    preallocated arrays), `with_lists_us` adds the binding's conversion of the
    plan into Python tuples."""
    import random

    import torch

    import positions_aware_cached_amd as pac

    S, C = 64, 1024
    K = torch.empty((S, C, 1, 64), dtype=torch.bfloat16, device="cuda")
    cache = pac.Cache.wrap([K], [torch.empty_like(K)])
    sched = pac.Scheduler(cache)
    rng = random.Random(0)
    next_id, spent, spent_lists, n_adm, n_ret = 0, 0.0, 0.0, 0, 0
    for i in range(args.sched_boundaries):
        while sched.counts()[0] < 8:
            sched.submit(next_id, rng.randint(128, 512), rng.randint(64, 256))
            next_id += 1
        t0 = time.perf_counter()
        sched.boundary_native()
        t1 = time.perf_counter()
        admitted, decode, retired = sched.last_plan()
        spent += t1 - t0
        spent_lists += time.perf_counter() - t0
        n_adm += len(admitted)
        n_ret += len(retired)
        for _, row, prompt in admitted:
            cache.set_row_length(row, prompt)
        for _, row, pos in decode:
            cache.set_row_length(row, pos + 1)
    us = spent / args.sched_boundaries * 1e6
    return {"slots": S, "boundaries": args.sched_boundaries, "boundary_us": round(us, 2),
            "with_lists_us": round(spent_lists / args.sched_boundaries * 1e6, 2),
            "admitted": n_adm, "retired": n_ret,
            "fraction_of_decode_step": round(us * 1e-3 / step_ms, 4)}


def bench_graph(args, cache, inp, pos, rows, out, ws, mirror, cfg, kv_bytes):
    """The same step replayed from a HIP graph: one graph holds the decode
    calls of all rotated layers (as a model's decode step would), so the
    launch gaps between steps disappear.  Timed over whole replays."""
    import torch
    import positions_aware_cached_amd as pac
    L = args.layers
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def step_all_layers():
        for layer in range(L):
            pac.decode_rope_store_attn(cache, layer, inp["q"], inp["k_new"], inp["v_new"], pos,
                                       rows, out, ws, cfg["base"], host_mirror=mirror,
                                       waves=args.waves, kernel=args.kernel)
    with torch.cuda.stream(side):
        step_all_layers()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_all_layers()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = args.graph_reps
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / (reps * L)
    return {"ms_per_step": round(ms, 4), "value": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "unit": "GB/s", "layers_per_graph": L, "replays": reps}


def prefill_label(name):
    """Workload name of a prefill leg, with its sizes."""
    import workloads
    cfg = workloads.config(name)
    if name == "chunk":
        starts, lens, _ = workloads.draw_chunk_meta(cfg)
        return (f"chunk_{cfg['A']}x{int(lens.min())}-{int(lens.max())}_at_{int(starts.min())}-"
                f"{int(starts.max())}")
    return f"prefill_{cfg['A']}x{cfg['T']}"


def bench_prefill(args, hip, name, K, dtype="bf16"):
    """Batched prefill, 32/8/128: "prefill" = 16 prompts x 1024 tokens into
    empty rows; "chunk" = 16 rows appending chunks of 128..512 tokens at starts
    in [0, 3072].  The attention kernel's own duration comes from events
    stamped in its dispatch; the store kernel runs before it in every step."""
    import torch

    import positions_aware_cached_amd as pac
    import workloads

    cfg = workloads.config(name, dtype=dtype)
    A, T, Hq, Hkv, D = (cfg[k] for k in ("A", "T", "Hq", "Hkv", "D"))
    inp = workloads.draw_prefill(cfg, device="cuda")
    cache = pac.Cache.wrap([inp["Kc"]], [inp["Vc"]])
    label = prefill_label(name)
    if name == "chunk":
        starts, lens, rows_h = workloads.draw_chunk_meta(cfg)
        meta_h = np.concatenate([starts, lens, rows_h]).astype(np.int32)
        meta = torch.as_tensor(meta_h, device="cuda")
    else:
        rows_h = inp["rows"]
        starts, lens = np.zeros(A, dtype=np.int64), np.full(A, T, dtype=np.int64)
    rows = torch.as_tensor(rows_h, device="cuda")
    out = torch.empty_like(inp["q"])
    ws = torch.empty(max(256, pac.prefill_workspace_size(cache, A, T, Hq)), dtype=torch.uint8,
                     device="cuda")
    evs = []
    for _ in range(K):
        pair = (ctypes.c_void_p * 2)()
        for j in range(2):
            h = ctypes.c_void_p()
            assert timing_event(hip, h) == 0
            pair[j] = h.value
        evs.append(pair)

    def step(ev=None):
        if name == "chunk":
            pac.prefill_chunk_rope_store_attn(cache, 0, inp["q"], inp["k_new"], inp["v_new"],
                                              meta, meta_h, out, ws, cfg["base"], attn_events=ev)
            return
        for r in rows_h:
            cache.reset_row(int(r))
        pac.prefill_rope_store_attn(cache, 0, inp["q"], inp["k_new"], inp["v_new"], rows, rows_h,
                                    out, ws, cfg["base"], attn_events=ev)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K
    ms = []
    for pair in evs:
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(pair[0]),
                                       ctypes.c_void_p(pair[1])) == 0
        ms.append(f.value)
        hip.hipEventDestroy(ctypes.c_void_p(pair[0]))
        hip.hipEventDestroy(ctypes.c_void_p(pair[1]))
    attn_ms = float(np.mean(ms))
    s64, n64 = starts.astype(np.float64), lens.astype(np.float64)
    # query t of entry a sees s_a + t + 1 keys: QK^T and PV, 2 flops per MAC
    flops = 4.0 * D * Hq * float(np.sum(n64 * s64 + n64 * (n64 + 1) / 2.0))
    tokens = float(np.sum(n64))
    hbm = (tokens * Hq * D * 2 * 2                           # q read, out written
           + 2 * tokens * Hkv * D * 2 * 2                    # k/v read, K/V stored
           + 2 * float(np.sum(s64)) * Hkv * D * 2)           # cached prefix K/V read once
    tflops = flops / (attn_ms * 1e-3) / 1e12
    return {"workload": label, "A": A, "T": T, "h_q": Hq, "h_kv": Hkv, "head_dim": D,
            "tokens": int(tokens), "ms_per_step": round(wall * 1e3, 4),
            "attn_kernel_ms": round(attn_ms, 4), "causal_gflop": round(flops / 1e9, 2),
            "tokens_per_s": round(tokens / wall, 1),
            "roofline": {"kernel": "k_prefill_mfma", "bound": "mfma",
                         "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("k_prefill_mfma", label)
                         if dtype == "bf16" else None},
            "hbm_gbs_step": round(hbm / wall / 1e9, 1)}


def cpu_model():
    """Model name of the host CPU (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_threads():
    """Worker threads for the all-core oracle runs: the host's CPUs, at most 16
    (the CPU share of one GPU on the measurement hosts)."""
    return max(1, min(16, os.cpu_count() or 1))


def cpu_baseline(args, cfg, inp, layers, pos_h, rows_h, out_gpu):
    """The CPU oracle, as it stands, on bounded samples of the same workload.

    Single thread: entries one by one, each on a host copy of its row's prefix,
    layer after layer of the rotated caches, until --cpu-seconds of oracle time.
    All cores: the same entries again, `oracle_threads()` at a time from a
    thread pool (the oracle's C entry point runs without the GIL); only the
    oracle calls are timed.  The layer-0 outputs are compared with the GPU's
    layer-0 outputs.  Then the prefill oracle on a stated sample of the
    16 x 1024 prefill, on one thread and on the pool."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import workloads

    Hkv, D = cfg["Hkv"], cfg["D"]
    qb, kb, vb = (workloads.bits(inp[k]) for k in ("q", "k_new", "v_new"))
    orc = oracle.default()
    if cfg["dtype"] == "f16":
        widen = lambda b: np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)
    else:
        widen = oracle.bf16_to_f32
    done, kv, elapsed, worst = [], 0, 0.0, 0.0
    t_start = time.perf_counter()
    out_bits = workloads.bits(out_gpu)

    def prefix(layer, a):
        Kc, Vc = layers[layer]
        p, r = int(pos_h[a]), int(rows_h[a])
        Km = workloads.bits(Kc[r, :p + 1]).reshape(1, p + 1, Hkv, D).copy()
        Vm = workloads.bits(Vc[r, :p + 1]).reshape(1, p + 1, Hkv, D).copy()
        return Km, Vm

    def run(a, Km, Vm):
        p = int(pos_h[a])
        return orc.decode_step(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], [p], [0], Km, Vm,
                               cfg["base"], dtype=cfg["dtype"])

    for layer in range(len(layers)):
        for a in range(len(pos_h)):
            Km, Vm = prefix(layer, a)
            t0 = time.perf_counter()
            o = run(a, Km, Vm)
            elapsed += time.perf_counter() - t0
            done.append((layer, a))
            kv += (int(pos_h[a]) + 1) * Hkv * D * 2 * 2
            if layer == 0:
                worst = max(worst, float(np.abs(widen(o[0]).astype(np.float64) -
                                                widen(out_bits[a]).astype(np.float64)).max()))
            if elapsed >= args.cpu_seconds or time.perf_counter() - t_start > 3 * args.cpu_seconds:
                break
        else:
            continue
        break

    nthr = oracle_threads()
    par = 0.0
    with ThreadPoolExecutor(max_workers=nthr) as pool:
        for c0 in range(0, len(done), nthr):
            batch = [(a,) + prefix(layer, a) for layer, a in done[c0:c0 + nthr]]
            t0 = time.perf_counter()
            list(pool.map(lambda x: run(*x), batch))
            par += time.perf_counter() - t0
    n = len(done)
    pf = prefill_oracle_sample(nthr)
    return {"value": round(kv / par / 1e9, 4), "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": f"{n} entry-steps of the {args.workload} decode step ({len(pos_h)} entries "
                      f"per layer, layers 0..{(n - 1) // len(pos_h)} of the rotated caches), {kv} "
                      f"KV bytes; {nthr} threads each calling the unchanged single-threaded "
                      f"oracle on one entry, {par:.2f} s of oracle calls",
            "tokens_per_s": round(n / par, 3),
            "single_thread": {"value": round(kv / elapsed / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "seconds": round(elapsed, 2),
                              "tokens_per_s": round(n / elapsed, 3)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "gpu_vs_oracle_max_abs": worst,
            "prefill": pf}


def prefill_oracle_sample(nthr):
    """The prefill oracle on the 16 x 1024 prefill configuration, sampled: every
    8th query (t = 7, 15, ..., 1023; each over its t + 1 keys, all 32 query
    heads, after storing all 1024 tokens), row 0 on one thread, then all 16
    rows on the thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import workloads

    cfg = workloads.config("prefill")
    A, T, Hq, D = cfg["A"], cfg["T"], cfg["Hq"], cfg["D"]
    inp = workloads.draw_prefill(cfg, device="cuda")
    qb, kb, vb = (workloads.bits(inp[k]) for k in ("q", "k_new", "v_new"))
    Kc, Vc = workloads.bits(inp["Kc"]).copy(), workloads.bits(inp["Vc"]).copy()
    rows = np.asarray(inp["rows"], dtype=np.int32)
    del inp
    t_list = np.arange(7, T, 8, dtype=np.int32)
    orc = oracle.default()
    flops_row = 4.0 * D * Hq * float(np.sum(t_list.astype(np.float64) + 1.0))

    def row(a):
        orc.prefill(qb[a:a + 1], kb[a:a + 1], vb[a:a + 1], rows[a:a + 1], Kc, Vc, cfg["base"],
                    t_list=t_list)

    t0 = time.perf_counter()
    row(0)
    one = time.perf_counter() - t0
    with ThreadPoolExecutor(max_workers=nthr) as pool:
        t0 = time.perf_counter()
        list(pool.map(row, range(A)))
        allr = time.perf_counter() - t0
    return {"workload": f"prefill_{A}x{T}", "unit": "GFLOP/s",
            "sample": f"queries t = 7, 15, ..., {T - 1} of each row (every 8th, each over its "
                      f"t + 1 keys, {Hq} query heads), after the store of all {T} tokens; "
                      f"{flops_row / 1e9:.2f} GFLOP of attention per row",
            "single_thread": {"rows": 1, "seconds": round(one, 2),
                              "value": round(flops_row / one / 1e9, 3)},
            "all_cores": {"rows": A, "threads": nthr, "seconds": round(allr, 2),
                          "value": round(A * flops_row / allr / 1e9, 3)}}


if __name__ == "__main__":
    main()
