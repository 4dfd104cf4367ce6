"""Benchmark of the token-level selection path on one MI355X.

One step = the whole hot path over one batch of the SnapKV/H2O-style workload
(36 layers x 8 KV heads x 32768 cached tokens x head dim 128, bf16 K/V, a
64-query window over 32 query heads): the LSE pass, the score pass (softmax
probabilities recovered from the LSE, summed over the GQA group and the
window), max-pool 7 fused into a per-(layer, KV head) top-8192 selection with
4 sink + 256 recent entries forced, and the gather of the kept K and V rows
into a compact cache.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.

Prints one JSON line.  Per-stage times come from HIP events recorded on the
stream the library launches on; every stage except the LSE pass (a partial
kernel plus a small combine kernel) and select (a key-preparation kernel
plus the per-unit selection kernel) is one kernel launch, so its stage time
is that kernel's launch duration.

Other modes:
  --copy-calib         a plain elementwise copy of 1 GiB (5 launches), to scale
                       the FETCH_SIZE / WRITE_SIZE counters to bytes
  --traffic-summary    turns four rocprofv3 --pmc CSV directories (kernel run
                       with FETCH_SIZE, with WRITE_SIZE; copy run with each)
                       into profiles/traffic_<kernel>.json
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "scored KV tokens/s & HBM GB/s vs peak; per-step select+gather latency"
COPY_BYTES = 1 << 30

# stage -> (kernel symbol stem, source file)
KERNELS = {"lse": ("lse_mfma_kernel", "k_window.hip"), "score": ("scores_mfma_kernel", "k_window.hip"),
           "select": ("select_kernel", "k_select.hip"), "gather": ("gather_rows_kernel", "k_gather.hip")}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the oracle sample for the CPU baseline")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--command", default="", help="profiling commands recorded in the traffic summary")
    return ap.parse_args()


def _source_sha(name):
    path = os.path.join(ROOT, "selection_score_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel, source):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % kernel)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != _source_sha(source):
        return None
    return t.get("bytes_per_launch")


def _copy_pair(device):
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=device)
    a.fill_(1.0)
    return a, torch.empty_like(a)


def copy_calibration():
    """5 launches of an elementwise copy (torch.neg) reading and writing 1 GiB each."""
    import torch
    a, b = _copy_pair("cuda:0")
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES, "copy_calibration_bytes_written": COPY_BYTES,
                      "launches": 5, "kernel": "elementwise neg, float32"}))


def copy_reference(stream):
    """Achievable-bandwidth reference measured in the same run: an elementwise
    copy of 1 GiB (read + write = 2 GiB of traffic), best of 5."""
    import torch
    a, b = _copy_pair("cuda:0")
    torch.neg(a, out=b)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.neg(a, out=b)
        e1.record(stream)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del a, b
    return 2 * COPY_BYTES / (best * 1e-3) / 1e9


def _counter_per_dispatch(d, counter):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 CSV directory."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        acc = {}
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name), v in acc.items():
            per.setdefault(name, []).append(v)
    return per


def traffic_summary(dirs, command):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel, scaled by
    what the same counter reads for the 1 GiB copy, written per kernel to
    profiles/traffic_<kernel>.json."""
    fetch, write, cfetch, cwrite = (_counter_per_dispatch(d, c) for d, c in
                                    zip(dirs, ["FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE"]))

    def copy_kib(per):
        vals = [v for n, vs in per.items() if "elementwise" in n.lower() for v in vs]
        vals = [v for v in vals if v > 0.5 * COPY_BYTES / 1024]    # the 1 GiB launches only
        return statistics.median(vals)

    f_scale = (COPY_BYTES / 1024) / copy_kib(cfetch)
    w_scale = (COPY_BYTES / 1024) / copy_kib(cwrite)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for stage, (stem, src) in KERNELS.items():
        names = [n for n in fetch if stem in n]
        if not names:
            continue
        fk = statistics.median(v for n in names for v in fetch[n])
        wk = statistics.median(v for n in names for v in write.get(n, [0.0]))
        rec = {"kernel": stem, "source": "selection_score_amd/csrc/" + src, "source_sha": _source_sha(src),
               "fetch_kib_raw": fk, "write_kib_raw": wk,
               "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
               "bytes_per_launch": (fk * f_scale + wk * w_scale) * 1024,
               "fetch_bytes": fk * f_scale * 1024, "write_bytes": wk * w_scale * 1024,
               "command": command}
        with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % stem), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))


def cpu_baseline(inp, cfg, seconds):
    """The oracle (window scores, max-pool, select, gather) on whole units,
    taken in a seeded order until the time budget is spent."""
    import numpy as np
    from oracle import materialise as om
    from oracle import numerics
    from oracle import score as osc
    from oracle import select as osel
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:                               # pragma: no cover
        limiter = None
    order = np.random.default_rng(cfg.seed).permutation(cfg.U)
    done, busy = 0, 0.0
    for u in order:
        l, g = divmod(int(u), cfg.Hkv)
        heads = slice(g * cfg.G, (g + 1) * cfg.G)
        q = inp["q"][l:l + 1, heads].float().cpu().numpy().astype(np.float64)
        k = inp["k"][l:l + 1, g:g + 1].float().cpu().numpy().astype(np.float64)
        v = inp["v"][l, g].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        a, _ = osc.window_scores(q, k)
        pooled = osc.pool1d(a[0, 0], cfg.pool, cfg.pool_k)
        kept, _ = osel.select_topk(numerics.round_to_f32(pooled), cfg.k, cfg.n_sink, cfg.n_recent)
        om.gather_view(k[0, 0], v, kept, 1)
        busy += time.perf_counter() - t0
        done += 1
        if busy >= seconds:
            break
    del limiter
    return {"value": done * cfg.N / busy, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d (layer, KV head) units in seeded order, full N=%d each: window scores "
                      "(LSE computed), max-pool, top-k, gather; %.1f s of oracle time, input copies "
                      "excluded" % (done, cfg.U, cfg.N, busy)}


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only; a run on several GPUs is not built "
              "(the (layer, KV head) units would shard across GPUs without any exchange)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, args.command)
        return
    if args.copy_calib:
        copy_calibration()
        return
    import torch
    import selection_score_amd as kv
    from selection_score_amd import workloads as wl

    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS["snapkv"]
    inp = wl.snapkv_inputs(cfg, dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    U, N, D = cfg.U, cfg.N, cfg.D
    lse = torch.empty((cfg.L, cfg.Hq, cfg.W), dtype=torch.float32, device=dev)
    scores = torch.empty((U, N), dtype=torch.float32, device=dev)
    kept = torch.empty((U, cfg.k), dtype=torch.int32, device=dev)
    dk = torch.empty((U, cfg.k, D), dtype=k.dtype, device=dev)
    dv = torch.empty_like(dk)
    k3, v3 = k.view(U, N, D), v.view(U, N, D)
    ws = kv.score_window(q, k, None, lse_out=lse)          # sizes and keeps the LSE workspace
    sel_ws = kv.select(scores, kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                       pool=cfg.pool, pool_k=cfg.pool_k)       # sizes and keeps the select workspace
    stream = torch.cuda.current_stream()
    copy_gbps = copy_reference(stream)

    def step(ev):
        ev[0].record(stream)
        kv.score_window(q, k, None, lse_out=lse, workspace=ws)
        ev[1].record(stream)
        kv.score_window(q, k, scores, lse_in=lse)
        ev[2].record(stream)
        kv.select(scores, kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  pool=cfg.pool, pool_k=cfg.pool_k, workspace=sel_ws)
        ev[3].record(stream)
        kv.gather_rerope(k3, v3, kept, dk, dv, bt=1, D=D, src_rows=N, src_unit_stride=N * D)
        ev[4].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for _ in range(args.warmup):
        step(warm)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    names = ["lse", "score", "select", "gather"]
    per = {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(names)}
    stage = {n: sum(t) / len(t) for n, t in per.items()}

    # algorithmic bytes per launch of each stage
    kb = cfg.L * cfg.Hkv * N * D * k.element_size()
    qb = q.numel() * q.element_size()
    sb = U * N * 4
    lb = lse.numel() * 4
    kept_b = U * cfg.k * 4
    gb = 2 * 2 * U * cfg.k * D * k.element_size()
    algo = {"lse": kb + qb + lb, "score": kb + qb + lb + sb, "select": sb + kept_b, "gather": kept_b + gb}
    step_bytes = sum(algo.values())
    # the roofline covers the slowest single-launch stage
    dom = max(["score", "gather"], key=lambda n: stage[n])
    achieved = algo[dom] / (stage[dom] * 1e-3) / 1e9
    tokens = cfg.L * cfg.Hkv * N
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "snapkv-h2o token scoring: 36 layers x 8 KV heads (32 query heads) x "
                               "32768 tokens x D128 bf16, window 64, max-pool 7, top 8192 per (layer, KV "
                               "head) with 4 sink + 256 recent, gather K+V",
                   "units": U, "tokens_per_unit": N, "budget": cfg.k},
        "stages_ms": stage,
        "stages_ms_median": {n: statistics.median(t) for n, t in per.items()},
        "stages_ms_min": {n: min(t) for n, t in per.items()},
        "stage_gbps": {n: algo[n] / (stage[n] * 1e-3) / 1e9 for n in names},
        "score_pass_tokens_per_s": tokens / (stage["score"] * 1e-3),
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "select_gather_ms": stage["select"] + stage["gather"],
        "copy_reference_gbps": copy_gbps,
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom][0], "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": _traffic(*KERNELS[dom]), "algorithmic_bytes": algo[dom],
                     "launch_ms": stage[dom]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
