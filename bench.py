"""Benchmark of the token-level selection path on one MI355X.

One step = the whole hot path over one batch of the SnapKV/H2O-style workload
(36 layers x 8 KV heads x 32768 cached tokens x head dim 128, bf16 K/V, a
64-query window over 32 query heads): the LSE pass, the score pass (softmax
probabilities recovered from the LSE, summed over the GQA group and the
window), max-pool 7 fused into a per-(layer, KV head) top-8192 selection with
4 sink + 256 recent entries forced, and the gather of the kept K and V rows
into a compact cache.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.

Prints one JSON line (see the design doc for every field).  Per-stage times come
from HIP events recorded on the stream the library launches on.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "scored KV tokens/s & HBM GB/s vs peak; per-step select+gather latency"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=12,
                    help="selection units the oracle processes for the CPU baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
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


def copy_calibration():
    import torch
    n = 1 << 30                                    # 1 GiB read + 1 GiB written
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def cpu_baseline(inp, cfg, n_units):
    """The oracle (score, pool, select, gather) on a bounded sample of units."""
    import numpy as np
    from oracle import materialise as om
    from oracle import numerics
    from oracle import score as osc
    from oracle import select as osel
    try:
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=cores)
    except Exception:                               # pragma: no cover
        cores, limiter = os.cpu_count(), None
    units = np.linspace(0, cfg.U - 1, n_units).astype(int)
    data = []
    for u in units:
        l, g = divmod(int(u), cfg.Hkv)
        heads = slice(g * cfg.G, (g + 1) * cfg.G)
        data.append((inp["q"][l:l + 1, heads].float().cpu().numpy().astype(np.float64),
                     inp["k"][l:l + 1, g:g + 1].float().cpu().numpy().astype(np.float64),
                     inp["v"][l, g].float().cpu().numpy().astype(np.float64)))
    t0 = time.perf_counter()
    for q, k, v in data:
        a, _ = osc.window_scores(q, k)
        pooled = osc.pool1d(a[0, 0], cfg.pool, cfg.pool_k)
        kept, _ = osel.select_topk(numerics.round_to_f32(pooled), cfg.k, cfg.n_sink, cfg.n_recent)
        om.gather_view(k[0, 0], v, kept, 1)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": n_units * cfg.N / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d (layer, KV head) units, full N=%d each: window scores, max-pool, "
                      "top-k, gather; %.1f s" % (n_units, cfg.U, cfg.N, dt)}


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(per-(layer, KV head) units shard without exchange; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
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
    stream = torch.cuda.current_stream()

    def step(ev):
        ev[0].record(stream)
        kv.score_window(q, k, None, lse_out=lse, workspace=ws)
        ev[1].record(stream)
        kv.score_window(q, k, scores, lse_in=lse)
        ev[2].record(stream)
        kv.select(scores, kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  pool=cfg.pool, pool_k=cfg.pool_k)
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
    stage = {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / args.steps for i, n in enumerate(names)}

    # algorithmic bytes per launch of each stage
    kb = cfg.L * cfg.Hkv * N * D * k.element_size()
    qb = q.numel() * q.element_size()
    sb = U * N * 4
    lb = lse.numel() * 4
    kept_b = U * cfg.k * 4
    gb = 2 * 2 * U * cfg.k * D * k.element_size()
    algo = {"lse": kb + qb + lb, "score": kb + qb + lb + sb, "select": sb + kept_b, "gather": kept_b + gb}
    step_bytes = sum(algo.values())
    kernel_of = {"lse": ("lse_mfma_kernel", "k_window.hip"), "score": ("scores_mfma_kernel", "k_window.hip"),
                 "select": ("select_kernel", "k_select.hip"), "gather": ("gather_rows_kernel", "k_gather.hip")}
    dom = max(["lse", "score", "gather"], key=lambda n: stage[n])
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
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "select_gather_ms": stage["select"] + stage["gather"],
        "roofline": {"bound": "hbm", "kernel": kernel_of[dom][0], "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": _traffic(*kernel_of[dom]), "algorithmic_bytes": algo[dom]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_units)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
