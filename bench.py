"""Benchmark of the MISA indexer decode step on one MI355X.

One step = the fused indexer call (router, routed scoring, top-k) for every
query of the workload (decode at 128K context: 16 sequences of 131072 keys,
one query each, H_I = 64, B = 128, h = 8, k = 2048), inputs resident in HBM.
Block pooling runs once per key cache and is timed separately.  The default
run also measures the plain streaming-read peak and, as `secondary`, the
prefill chunk (4096 queries over 65536 keys, MFMA-bound).  Prints one JSON
line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-secondary]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MISA indexer us per decode batch at L=128K; key-scores/s; % of HBM/MFMA roof"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KEY_BYTES = 128 * 2  # one bf16 indexing key
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "long_context_sparse_05_amd", "csrc", f)
                  for f in ("score.hip", "common.hpp", "select.hpp", "route_finish.hpp")]


class HipEvents:
    """Raw hipEvent_t handles (the scoring kernel is timed on the stream it
    is launched on, from inside the library's launch sequence)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        assert self.hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return out.value


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per scoring launch from the committed rocprofv3 counter runs,
    or None when absent or taken on a different kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("kernel_hash") != kernel_hash():
        return None
    return ent.get("bytes_per_launch")


COPY_MIB = 512


def copy_calibration():
    """A plain device copy of known size (COPY_MIB MiB read, COPY_MIB MiB
    written), run under rocprofv3 --pmc to scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.empty(COPY_MIB << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_MIB << 20, "launches": 3}), flush=True)
    return 0


def _counter_rows(path):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_kernel_kib(rows, counter, name_part):
    """Mean counter value per dispatch of the kernels whose name contains
    name_part."""
    vals = [float(r["Counter_Value"]) for r in rows
            if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", "")]
    return sum(vals) / len(vals) if vals else None


def summarize_counters(workload, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """Write the scoring kernel's HBM traffic per launch (FETCH_SIZE and
    WRITE_SIZE, each scaled by the same counter on the plain copy of known
    size) to profiles/score_kernel_traffic.json, keyed by the kernel-source
    hash so a changed kernel reads as unmeasured."""
    # the fused call's scoring kernel (router reduce in its prologue), the one
    # the headline's roofline times -- not the separate-call or dense variants
    kname = "score_rows_kernel<1, false, true,"
    f_k = _per_kernel_kib(_counter_rows(fetch_dir), "FETCH_SIZE", kname)
    w_k = _per_kernel_kib(_counter_rows(write_dir), "WRITE_SIZE", kname)
    # the runtime's device copy kernel moves the known bytes (torch's fill of
    # the source buffer is a separate, small dispatch)
    f_c = _per_kernel_kib(_counter_rows(cfetch_dir), "FETCH_SIZE", "copyBuffer")
    w_c = _per_kernel_kib(_counter_rows(cwrite_dir), "WRITE_SIZE", "copyBuffer")
    copy_kib = (COPY_MIB << 20) / 1024.0
    fs = copy_kib / f_c if f_c else None
    wsf = copy_kib / w_c if w_c else None
    rec = {}
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
    ent = {"kernel_hash": kernel_hash(), "fetch_kib_raw": f_k, "write_kib_raw": w_k,
           "copy_fetch_kib_raw": f_c, "copy_write_kib_raw": w_c,
           "fetch_scale": fs, "write_scale": wsf}
    if f_k is not None and w_k is not None and fs and wsf:
        ent["bytes_per_launch"] = (f_k * fs + w_k * wsf) * 1024.0
    rec[workload] = ent
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(ent), flush=True)
    return 0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_rows(case, cfg, rows, reps=3, threads=None):
    """The oracle on the query rows `rows` of the workload, median of `reps`
    runs (`threads`: OpenMP threads, default all).  Returns (key-scores/s,
    threads used, outputs of the last run)."""
    import numpy as np
    from oracle import oracle as orc
    sub = dict(case)
    for key in ("q", "w", "q_seq", "q_pos"):
        sub[key] = np.ascontiguousarray(case[key][rows])
    b = orc.Batch.from_case(sub)
    kind = cfg["kind"]
    before = orc.num_threads()
    if threads:
        orc.set_num_threads(threads)
    times = []
    out = None
    try:
        for _ in range(reps):
            t0 = time.perf_counter()
            if kind == "dagger":
                out = orc.misa_dagger(b, cfg["B"], cfg["h"], cfg["kc"], cfg["k"])
            elif kind == "hisa":
                out = orc.hisa(b, cfg["B"], cfg["m"], cfg["k"])
            elif kind == "misa_hisa":
                heads, _ = orc.route(b, cfg["B"], cfg["h"])
                out = orc.hisa(b, cfg["B"], cfg["m"], cfg["k"], heads=heads)
                out["heads"] = heads
            elif "h" in cfg:
                out = orc.misa(b, cfg["B"], cfg["h"], cfg["k"])
            else:
                idx, _ = orc.dsa(b, cfg["k"])
                out = {"idx": idx}
            times.append(time.perf_counter() - t0)
        used = orc.num_threads()
    finally:
        orc.set_num_threads(before)
    n = float((sub["q_pos"].astype(np.int64) + 1).sum())
    return n / float(np.median(times)), used, out


READ_PEAK_MIB = 512


def measure_read_peak(ev, reps=10):
    """The plain streaming read (misa_stream_read) of a 512 MiB buffer after a
    1 GiB fill that evicts the caches, at 512 workgroups (two per CU, as the
    decode scoring kernel): median and spread of `reps` event-timed runs."""
    import numpy as np
    import torch
    from long_context_sparse_05_amd import abi
    nbytes = READ_PEAK_MIB << 20
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    wgs = 512
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    for _ in range(3):
        abi.stream_read(buf, wgs, sink)
    us = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        e0, e1 = ev.create(), ev.create()
        abi.stream_read(buf, wgs, sink, events=(e0, e1))
        torch.cuda.synchronize()
        us.append(ev.ms(e0, e1) * 1e3)
    del buf, flush
    gbs = [nbytes / u / 1e3 for u in us]
    return {"GBs_median": float(np.median(gbs)), "GBs_p10_p90": [float(np.percentile(gbs, 10)),
                                                                 float(np.percentile(gbs, 90))],
            "bytes": nbytes, "workgroups": wgs, "kernel": "stream_read_kernel (misa_stream_read)",
            "method": "event-timed, each run after a 1 GiB fill evicting L2 and the MALL"}


def measure(workload, K, W, ev, cpu=True, cpu_rows_cap=None):
    """One workload: warm-up, K back-to-back steps (the headline), the scoring
    kernel's own duration, separate calls, cold single steps, CPU baseline and
    a parity summary.  Returns the result fields."""
    import numpy as np
    import torch
    from long_context_sparse_05_amd import abi, synth

    case, cfg = synth.make_workload(workload, seed=0)
    kind = cfg["kind"]
    routed = "h" in cfg
    hier = kind in ("hisa", "misa_hisa")  # the hierarchical indexer's step
    B, h, k = cfg.get("B"), cfg.get("h"), cfg["k"]
    kc = cfg.get("kc", k)
    m = cfg.get("m")
    b = abi.Batch.from_numpy(case)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    dev = "cuda"

    pool_us = None
    pooled = None
    if B is not None:  # once per key cache: block pooling
        pooled = abi.pool(b, B)
        e0, e1 = ev.create(), ev.create()
        ev.record(e0, sp)
        for _ in range(3):
            abi.pool(b, B, out=pooled)
        ev.record(e1, sp)
        pool_us = ev.ms(e0, e1) / 3 * 1e3

    k1 = kc if kind == "dagger" else k  # selection size of the scoring call
    heads = torch.empty((b.T, h), dtype=torch.int32, device=dev) if routed else None
    idx = torch.empty((b.T, k1), dtype=torch.int32, device=dev)
    val = torch.empty((b.T, k1), dtype=torch.float32, device=dev)
    fin = torch.empty((b.T, k), dtype=torch.int32, device=dev)
    fin_val = torch.empty((b.T, k), dtype=torch.float32, device=dev)
    if hier:
        ws_h = b.workspace(abi.MISA_OP_HISA, B=B, h=h or 1, k=k, kc=m)
        ws_r = b.workspace(abi.MISA_OP_ROUTE, B=B, h=h) if routed else None
    elif routed:
        ws_i = b.workspace(abi.MISA_OP_INDEXER, B=B, h=h, k=k1)
        ws_r = b.workspace(abi.MISA_OP_ROUTE, B=B, h=h)
        ws_s = b.workspace(abi.MISA_OP_SCORE_TOPK, h=h, k=k1)
    else:
        ws_d = b.workspace(abi.MISA_OP_DENSE, k=k)
    ws_rr = b.workspace(abi.MISA_OP_RERANK, k=k, kc=kc) if kind == "dagger" else None

    def step(events=None):
        if hier:  # (router, then) block scores, kept blocks, refinement, top-k
            if routed:
                abi.route(b, pooled, B, h, 0, heads=heads, ws=ws_r)
            abi.hisa_indexer(b, pooled, B, m, k, heads=heads, idx=idx, val=val, ws=ws_h,
                             events=events)
        elif routed:  # the fused call: router, routed scoring, top-k (k' for MISA-dagger)
            abi.indexer(b, pooled, B, h, k1, heads=heads, idx=idx, val=val, ws=ws_i, events=events)
            if kind == "dagger":  # fine stage: all-head rescoring of the k' candidates
                abi.rerank(b, idx, k, idx=fin, val=fin_val, ws=ws_rr)
        else:  # the dense DSA indexer
            abi.score_topk(b, None, k, idx=idx, val=val, ws=ws_d, events=events)

    def step_separate():  # the routed step as separate calls
        abi.route(b, pooled, B, h, 0, heads=heads, ws=ws_r)
        abi.score_topk(b, heads, k1, idx=idx, val=val, ws=ws_s)
        if kind == "dagger":
            abi.rerank(b, idx, k, idx=fin, val=fin_val, ws=ws_rr)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    # the timed region: K whole steps, events only at its two ends
    t_start, t_stop = ev.create(), ev.create()
    wall0 = time.perf_counter()
    ev.record(t_start, sp)
    for _ in range(K):
        step()
    ev.record(t_stop, sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev.ms(t_start, t_stop) / K
    # the scoring kernel's own duration: a second pass of K steps with events
    # attached to that kernel's launch on its stream (the library stamps
    # them with the kernel's begin and end); kept out of the headline region
    sev = [(ev.create(), ev.create()) for _ in range(K)]
    for i in range(K):
        step(sev[i])
    torch.cuda.synchronize()
    score_ms = float(np.mean([ev.ms(a, c) for a, c in sev]))
    ms_sep = None
    if routed and not hier:
        for _ in range(W):
            step_separate()
        ev.record(t_start, sp)
        for _ in range(K):
            step_separate()
        ev.record(t_stop, sp)
        torch.cuda.synchronize()
        ms_sep = ev.ms(t_start, t_stop) / K
    # cold caches: before each step a 1 GiB fill evicts L2 and the 256 MB
    # MALL, and events bracket the step alone (reported beside the headline,
    # which times back-to-back steps)
    # context for several queries per sequence: the same routed rows scored
    # one by one (misa_score, which takes the per-row kernel), kernel time
    per_row_us = None
    if routed and cfg.get("queries_per_seq", 1) > 1 and b.S > 1:
        sc_rows = torch.empty((b.T, b.Lmax), dtype=torch.float32, device=dev)
        abi.score(b, heads, out=sc_rows)
        ev.record(t_start, sp)
        for _ in range(5):
            abi.score(b, heads, out=sc_rows)
        ev.record(t_stop, sp)
        torch.cuda.synchronize()
        per_row_us = ev.ms(t_start, t_stop) / 5 * 1e3
        del sc_rows
    # context only: the dense DSA indexer (every head, no routing) on the same
    # inputs and k, warm back-to-back steps like the headline
    dsa_us = None
    if routed and not hier and kind != "dagger":
        ws_dd = b.workspace(abi.MISA_OP_DENSE, k=k)
        di = torch.empty((b.T, k), dtype=torch.int32, device=dev)
        dv = torch.empty((b.T, k), dtype=torch.float32, device=dev)
        for _ in range(2):
            abi.score_topk(b, None, k, idx=di, val=dv, ws=ws_dd)
        nd = max(2, min(K, 5))
        ev.record(t_start, sp)
        for _ in range(nd):
            abi.score_topk(b, None, k, idx=di, val=dv, ws=ws_dd)
        ev.record(t_stop, sp)
        torch.cuda.synchronize()
        dsa_us = ev.ms(t_start, t_stop) / nd * 1e3
        del ws_dd, di, dv
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cev = [(ev.create(), ev.create()) for _ in range(K)]
    for i in range(K):
        flush.fill_(float(i))
        ev.record(cev[i][0], sp)
        step()
        ev.record(cev[i][1], sp)
    torch.cuda.synchronize()
    cold_all = np.array([ev.ms(a, c) for a, c in cev])
    del flush
    step()  # leave the fused call's outputs for the parity check
    torch.cuda.synchronize()

    n_keys = int((case["q_pos"].astype(np.int64) + 1).sum())
    value = n_keys / (ms_step * 1e-3)
    nh = h if routed else b.H
    if kind == "prefill":
        # dense MFMA contraction: 2 * 128 flops per (query, routed head, prefix key)
        flops = 2.0 * 128 * nh * n_keys
        achieved = flops / (score_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                "kernel": "score_prefill_kernel (32x32x16 bf16 MFMA, %d routed heads)" % nh,
                "alg_flops_per_launch": flops}
    elif hier:
        # the refinement kernel gathers the candidate keys of the kept blocks
        qp = case["q_pos"].astype(np.int64)
        n_cand = int(np.minimum(m * B, qp + 1).sum())
        alg_bytes = n_cand * KEY_BYTES + b.T * nh * KEY_BYTES
        achieved = alg_bytes / (score_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": "score_rows_kernel (gathered candidate rows, %d heads)" % nh,
                "alg_bytes_per_launch": alg_bytes}
    elif cfg.get("queries_per_seq", 1) > 1 and b.S > 1:
        # several queries per sequence: each sequence's keys are read once for
        # all its rows (its longest prefix), plus the routed query rows
        qp = case["q_pos"].astype(np.int64)
        seq_keys = sum(int(qp[case["q_seq"] == s_].max()) + 1 for s_ in range(b.S))
        alg_bytes = seq_keys * KEY_BYTES + b.T * nh * KEY_BYTES
        achieved = alg_bytes / (score_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": "score_prefill_kernel (multi-query tile table, %d routed heads)" % nh,
                "alg_bytes_per_launch": alg_bytes}
    else:
        alg_bytes = n_keys * KEY_BYTES + b.T * nh * KEY_BYTES  # keys streamed + query rows
        achieved = alg_bytes / (score_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(workload),
                "kernel": "score_rows_kernel (%d-row head tiles, direct rows)" % (16 * ((nh + 15) // 16)),
                "alg_bytes_per_launch": alg_bytes}

    res = {
        "ms_per_step": ms_step,
        "value": value,
        "config": {"workload": workload, "sequences": int(b.S), "context": int(b.Lmax),
                   "queries": int(b.T), "H_I": int(b.H), "B": B, "h": h, "k": k, "d": 128},
        "us_per_batch": ms_step * 1e3,
        # each cold step bracketed by its own events: median and spread
        "us_per_batch_cold_p10_p50_p90": [float(np.percentile(cold_all, q)) * 1e3 for q in (10, 50, 90)],
        "score_kernel_us": score_ms * 1e3,
        "wall_s_timed": wall,
        "roofline": roof,
    }
    if kind == "dagger":
        res["config"]["k_prime"] = kc
    if hier:
        res["config"]["kept_blocks"] = m
    if ms_sep is not None:
        res["us_per_batch_separate_calls"] = ms_sep * 1e3
    if per_row_us is not None:
        res["multi_query"] = {"shared_pass_scoring_us": score_ms * 1e3, "per_row_scoring_us": per_row_us,
                              "note": "the routed rows scored with a shared pass over each sequence's keys "
                                      "(the step) against one pass per row (misa_score)"}
    if dsa_us is not None:
        res["dsa_vs_misa"] = {"dsa_dense_us_per_step": dsa_us, "misa_us_per_step": ms_step * 1e3,
                              "dsa_over_misa": dsa_us / (ms_step * 1e3),
                              "note": "context, not a target: the dense indexer over all %d heads "
                                      "on the same inputs and k" % b.H}
    if pool_us is not None:
        res["pool_us_once_per_cache"] = pool_us
    if kind != "prefill" and not hier:
        # whole step: keys, complete pooled blocks and all head queries read;
        # selected ids and scores written
        n_blocks = int((case["q_pos"].astype(np.int64) // B).sum()) if routed else 0
        step_bytes = (n_keys * KEY_BYTES + n_blocks * 128 * 4 + b.T * b.H * (KEY_BYTES + 4)
                      + b.T * k1 * 8 + (b.T * kc * KEY_BYTES if kind == "dagger" else 0))
        res["hbm_frac_whole_step"] = step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    if cpu:
        if kind == "prefill":  # a bounded sample: 16 query rows spread over the chunk
            rows = np.linspace(0, b.T - 1, 16).astype(np.int64)
            sample = "16 of %d query rows (evenly spaced), median of 3 runs" % b.T
        else:
            rows = np.arange(b.T)
            sample = "all %d queries of the workload, median of 3 runs" % b.T
        cv, cores, out = cpu_baseline_rows(case, cfg, rows)
        # one thread on a smaller sample: two of the rows
        r1 = rows[:2]
        cv1, _, _ = cpu_baseline_rows(case, cfg, r1, reps=1, threads=1)
        res["cpu_baseline"] = {"value": cv, "unit": "key-scores/s", "cores": cores,
                               "kind": "oracle", "sample": sample, "cpu_model": cpu_model(),
                               "value_1thread": cv1, "sample_1thread": "%d query rows, one run" % len(r1)}
        gi = (fin if kind == "dagger" else idx).cpu().numpy()[rows]
        par = {"rows_checked": int(len(rows)),
               "set_overlap": float(np.mean([len(set(gi[i]) & set(out["idx"][i])) / k
                                             for i in range(len(rows))]))}
        if routed:
            gh = heads.cpu().numpy()[rows]
            par["heads_equal"] = bool(np.array_equal(np.sort(gh, 1), np.sort(out["heads"], 1)))
        res["parity_vs_oracle"] = par
    return res


SECONDARY = "misa_prefill_chunk_4096q_L65536"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="misa_decode_16x128K")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the prefill-chunk record of the default run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy of known size (for counter scaling)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="rocprofv3 --pmc output dirs of the bench and of --copy-calibration")
    args = ap.parse_args(argv)
    if args.summarize_counters:
        return summarize_counters(args.workload, *args.summarize_counters)
    if args.copy_calibration:
        return copy_calibration()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the indexer path here is built and timed on a single "
              "MI355X; %d GPUs (--gpus %d, WORLD_SIZE %d) is not supported"
              % (max(args.gpus, world), args.gpus, world), file=sys.stderr)
        return 2

    import torch
    from long_context_sparse_05_amd import abi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    abi.load()
    ev = HipEvents()
    K, W = args.steps, args.warmup
    peak = measure_read_peak(ev)
    r = measure(args.workload, K, W, ev, cpu=not args.no_cpu)
    roof = r["roofline"]
    if roof["bound"] == "hbm":
        roof["measured_read_peak_GBs"] = peak["GBs_median"]
        roof["frac_of_measured_read_peak"] = roof["achieved"] / peak["GBs_median"]
    res = {
        "metric": METRIC,
        "value": r.pop("value"),
        "unit": "key-scores/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": r.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    res.update(r)
    res["hbm_read_peak_measured"] = peak
    if args.workload != SECONDARY and not args.no_secondary:
        # the prefill chunk (MFMA-bound) beside the decode headline, fewer
        # steps; ten untimed steps first (its first few steps on fresh
        # buffers run about 10% slower than the steady state)
        s_k, s_w = min(K, 10), max(W, 10)
        s = measure(SECONDARY, s_k, s_w, ev, cpu=not args.no_cpu)
        s["steps"], s["warmup"] = s_k, s_w
        s["us_per_step"] = s.pop("ms_per_step") * 1e3
        s["key_scores_per_s"] = s.pop("value")
        for key in ("wall_s_timed", "us_per_batch"):
            s.pop(key, None)
        res["secondary"] = s
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
