"""Benchmark of the selection path on one MI355X.

The default workload is the largest configuration that fits one GPU, the
10M-token scale-out block retrieval: a Mean-K index of 64 layers x 8 KV heads
x 312500 32-token blocks (fp16, D 128) scored in 65536-block tiles for 4
sessions with independent 512-token queries, a running top-4096 per
(session, layer, KV head) with block 0 and the last 4 blocks forced, and the
in-place incremental update of each session's 4096-page view (about half the
blocks reused in their pages; moved ones and misses re-RoPEd from the
HBM-resident raw store at their new positions).  One step is all of that over one batch of seeded synthetic inputs
resident in HBM before timing starts.

Prints one JSON line.  Per-stage times come from HIP events recorded on the
stream the library launches on.  `roofline` covers the longest kernel of the
step; its stage time per launch also holds the short kernels the same library
call launches with it (listed as `companions`), so `achieved` is a lower
bound for the kernel alone.

--workload picks another workload: tiny (token-level eviction, 2 units of
2048 fp32 keys; latency with the caches flushed before every step), snapkv
(SnapKV/H2O-style window scoring with the LSE pass, max-pool, top-8192 per
unit, gather), intentkv (session memory over a paged pool with the dead-slot
redirect), kvmem1m (1M-token block retrieval and re-RoPE gather), meank1m
(building the Mean-K index of the 1M-token workspace), actkv (one ActKV
compression step: LRFU keep score, eviction by keep score, in-place tail
compaction), actkv_decode (one decode token of ActKV's recovery-based action
scorer over paged K).

`cpu_baseline` is the oracle (oracle/, NumPy float64) timed on this host's
cores over a bounded sample of the same workload; the sample is stated.

Other modes:
  --copy-calib         a plain elementwise copy of 1 GiB (5 launches), to scale
                       the FETCH_SIZE / WRITE_SIZE counters to bytes
  --traffic-summary    turns four rocprofv3 --pmc CSV directories (kernel run
                       with FETCH_SIZE, with WRITE_SIZE; copy run with each)
                       into profiles/traffic_<kernel>_<workload>.json
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "scored KV tokens/s & HBM GB/s vs peak; per-step select+gather latency"
COPY_BYTES = 1 << 30

# every kernel of the library -> its source file (traffic summaries)
KERNEL_SOURCES = {
    "lse_mfma_kernel": "k_window.hip", "lse_combine_kernel": "k_window.hip",
    "scores_mfma_kernel": "k_window.hip", "lse_valu_kernel": "k_window.hip",
    "scores_valu_kernel": "k_window.hip", "pool1d_kernel": "k_window.hip",
    "select_keys_kernel": "k_select.hip", "select_regs_kernel": "k_select.hip", "select_kernel": "k_select.hip",
    "slice_digit_kernel": "k_select.hip", "slice_count_kernel": "k_select.hip", "slice_place_kernel": "k_select.hip",
    "select_tile_kernel": "k_select_tile.hip",
    "gather_rows_kernel": "k_gather.hip", "gather_blocks_kernel": "k_gather.hip",
    "incremental_plan_kernel": "k_incremental.hip", "incremental_data_kernel": "k_incremental.hip",
    "memory_logits_kernel": "k_memory.hip", "memory_logits_mfma_kernel": "k_memory.hip",
    "memory_lse_kernel": "k_memory.hip",
    "memory_rule_kernel": "k_memory.hip", "memory_layer_sum_kernel": "k_memory.hip",
    "query_reduce_kernel": "k_block.hip", "block_scores_kernel": "k_block.hip",
    "block_scores_mfma_kernel": "k_block.hip",
    "memory_update_kernel": "k_misc.hip", "memory_update_vec_kernel": "k_misc.hip",
    "redirect_kernel": "k_misc.hip", "sentinel_kernel": "k_misc.hip",
    "mean_k_kernel": "k_index.hip",
    "free_clear_kernel": "k_misc.hip", "free_mark_kernel": "k_misc.hip", "free_compact_kernel": "k_misc.hip",
    "compact_plan_kernel": "k_compact.hip", "compact_copy_kernel": "k_compact.hip",
    "decode_score_kernel": "k_decode.hip", "action_reduce_kernel": "k_decode.hip",
    "top_p_update_kernel": "k_decode.hip",
}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the oracle sample for the CPU baseline")
    ap.add_argument("--workload", default="kvmem10m",
                    choices=["kvmem10m", "tiny", "snapkv", "intentkv", "kvmem1m", "meank1m", "actkv", "actkv_decode"],
                    help="which workload one step runs (the default line is kvmem10m)")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--command", default="", help="profiling commands recorded in the traffic summary")
    return ap.parse_args()


def _source_sha(name):
    """SHA-256 (16 hex digits) of the code of a kernel source and of every
    local header it includes, recursively (the package's csrc/, then
    include/), with comments and whitespace removed: an edit of the comments
    keeps the summaries that were taken on the same code."""
    import re
    h = hashlib.sha256()
    seen = set()
    comment = re.compile(rb'//[^\n]*|/\*.*?\*/', re.S)

    def add(n):
        if n in seen:
            return
        seen.add(n)
        for d in (os.path.join(ROOT, "selection_score_amd", "csrc"), os.path.join(ROOT, "include")):
            path = os.path.join(d, n)
            if os.path.exists(path):
                with open(path, "rb") as f:
                    data = f.read()
                code = re.sub(rb"\s+", b"", comment.sub(b" ", data))
                h.update(n.encode() + b"\0" + code)
                for inc in re.findall(rb'#include "([^"]+)"', data):
                    add(inc.decode())
                return
        raise FileNotFoundError(n)

    add(name)
    return h.hexdigest()[:16]


def _traffic(kernel, source, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != _source_sha(source):
        return None
    return t.get("bytes_per_launch")


def _kernels_traffic(kernels, workload):
    """Counter bytes of a list of (kernel, source) launches, summed (None
    unless every summary is current)."""
    vals = [_traffic(k, src, workload) for k, src in kernels]
    return None if any(v is None for v in vals) else sum(vals)


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


def traffic_summary(dirs, command, workload):
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
    import re
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    stems = {}
    for n in fetch:
        mt = re.search(r"kvsel::(\w+)", n)
        if mt and mt.group(1) in KERNEL_SOURCES:
            stems.setdefault(mt.group(1), []).append(n)
    for stem, names in sorted(stems.items()):
        src = KERNEL_SOURCES[stem]
        fk = statistics.median(v for n in names for v in fetch[n])
        wk = statistics.median(v for n in names for v in write.get(n, [0.0]))
        rec = {"kernel": stem, "source": "selection_score_amd/csrc/" + src, "source_sha": _source_sha(src),
               "workload": workload,
               "fetch_kib_raw": fk, "write_kib_raw": wk,
               "copy_scale_fetch": f_scale, "copy_scale_write": w_scale,
               "bytes_per_launch": (fk * f_scale + wk * w_scale) * 1024,
               "fetch_bytes": fk * f_scale * 1024, "write_bytes": wk * w_scale * 1024,
               "command": command}
        with open(os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (stem, workload)), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))


class OracleTimer:
    """Times the oracle (NumPy float64, test infrastructure) on this host for
    the cpu_baseline leg: BLAS threads on every core of the process's
    affinity mask; only the oracle's own calls are timed (copies of the
    inputs to the host and their conversion to float64 are not)."""

    def __init__(self, seconds):
        self.seconds = seconds
        self.cores = len(os.sched_getaffinity(0))
        self.busy = 0.0
        try:
            from threadpoolctl import threadpool_limits
            self._limiter = threadpool_limits(limits=self.cores)
        except Exception:                           # pragma: no cover
            self._limiter = None

    def run(self, fn, *a, **kw):
        t0 = time.perf_counter()
        out = fn(*a, **kw)
        self.busy += time.perf_counter() - t0
        return out

    def spent(self):
        return self.busy >= self.seconds

    def result(self, tokens, sample):
        return {"value": tokens / self.busy, "unit": "tokens/s", "cores": self.cores, "kind": "oracle",
                "sample": sample + "; %.1f s of oracle time, input copies excluded" % self.busy}


def _np64(t):
    """torch tensor (any dtype, any device) -> float64 NumPy array, exactly."""
    import numpy as np
    import torch
    x = t.detach().to("cpu")
    if x.dtype != torch.float64:
        x = x.to(torch.float32)
    return x.numpy().astype(np.float64)


class Tiny:
    """Token-level eviction at the tiny size (1 layer, 2 KV / 8 query heads,
    2048 fp32 keys of D 64, 16 planted high-norm keys): window scores over the
    last 16 queries with the LSE computed, top-512 per KV head of the avg-pool
    7 scores (pooled inside the select's workgroup) with 4 sink + 64 recent,
    gather of the kept K and V rows.  A latency measurement: before every
    step a 1 GiB fill evicts L2 and the Infinity Cache (outside the step's
    events), and ms_per_step is the mean of the steps' own event spans."""
    stages = ["score", "select", "gather"]
    dominant = ("score", [("lse_valu_kernel", "k_window.hip"), ("scores_valu_kernel", "k_window.hip")])
    score_stage = "score"
    materialise_stages = ["select", "gather"]
    dtype = "f32"
    flush = True

    def __init__(self, torch, kv, wl, dev):
        self.torch, self.kv, self.cfg = torch, kv, wl.CONFIGS["tiny"]
        cfg = self.cfg
        self.inp = wl.tiny_inputs(cfg, dev)
        U, N, D = cfg.U, cfg.N, cfg.D
        self.scores = torch.empty((U, N), dtype=torch.float32, device=dev)
        self.kept = torch.empty((U, cfg.k), dtype=torch.int32, device=dev)
        self.dk = torch.empty((U, cfg.k, D), dtype=torch.float32, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.k3, self.v3 = self.inp["k"].view(U, N, D), self.inp["v"].view(U, N, D)
        self.ws = kv.score_window(self.inp["q"], self.inp["k"], self.scores)
        self.sel_ws = kv.select(self.scores, self.kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                pool=cfg.pool, pool_k=cfg.pool_k)
        self.flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        self.tokens = cfg.L * cfg.Hkv * N

    def pre_step(self):
        self.flush_buf.fill_(1.0)

    def step(self, ev, stream, it):
        kv, cfg, inp = self.kv, self.cfg, self.inp
        ev[0].record(stream)
        kv.score_window(inp["q"], inp["k"], self.scores, workspace=self.ws)
        ev[1].record(stream)
        kv.select(self.scores, self.kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  pool=cfg.pool, pool_k=cfg.pool_k, workspace=self.sel_ws)
        ev[2].record(stream)
        kv.gather_rerope(self.k3, self.v3, self.kept, self.dk, self.dv, bt=1, D=cfg.D, src_rows=cfg.N,
                         src_unit_stride=cfg.N * cfg.D)
        ev[3].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        kb = cfg.U * cfg.N * cfg.D * 4
        qb = cfg.L * cfg.Hq * cfg.W * cfg.D * 4
        sb = cfg.U * cfg.N * 4
        kept_b = cfg.U * cfg.k * 4
        # the score call reads K twice (LSE pass, score pass) and writes the
        # scores; the select reads them and pools them in its workgroup
        return {"score": 2 * (kb + qb) + sb, "select": sb + kept_b,
                "gather": kept_b + 2 * 2 * cfg.U * cfg.k * cfg.D * 4}

    def cpu_baseline(self, seconds):
        """The whole step on the oracle, repeated: window scores with the LSE,
        avg-pool, top-512 per KV head, gather (bounded to ~1 s)."""
        from oracle import materialise as om
        from oracle import numerics
        from oracle import score as osc
        from oracle import select as osel
        cfg = self.cfg
        clock = OracleTimer(min(seconds, 1.0))
        q, k, v = _np64(self.inp["q"]), _np64(self.inp["k"]), _np64(self.inp["v"])
        reps = 0
        while not clock.spent():
            a, _ = clock.run(osc.window_scores, q, k)
            pooled = clock.run(osc.pool1d, a, cfg.pool, cfg.pool_k)
            for u in range(cfg.U):
                l, g = divmod(u, cfg.Hkv)
                kept, _ = clock.run(osel.select_topk, numerics.round_to_f32(pooled[l, g]), cfg.k, cfg.n_sink,
                                    cfg.n_recent)
                clock.run(om.gather_view, k[l, g], v[l, g], kept, 1)
            reps += 1
        return clock.result(reps * self.tokens, "%d repetitions of the whole step (%d units of %d keys)"
                            % (reps, cfg.U, cfg.N))

    def config(self):
        cfg = self.cfg
        return {"workload": "tiny token-level eviction: 1 layer x 2 KV heads (8 query heads) x 2048 tokens x "
                            "D64 fp32, window 16, avg-pool 7, top 512 per KV head with 4 sink + 64 recent, "
                            "gather K+V; caches flushed before every step",
                "units": cfg.U, "tokens_per_unit": cfg.N, "budget": cfg.k}

    def extra(self):
        return {}


class SnapKV:
    """Token scoring against a 64-query window: LSE pass, score pass, select
    (max-pool 7 fused), gather of the kept K and V rows."""
    stages = ["lse", "score", "select", "gather"]
    # the longest kernel and the launches of its stage (kernel first)
    dominant = ("lse", [("lse_mfma_kernel", "k_window.hip"), ("lse_combine_kernel", "k_window.hip")])
    score_stage = "score"
    materialise_stages = ["select", "gather"]
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.kv, cfg = kv, wl.CONFIGS["snapkv"]
        self.cfg = cfg
        self.inp = wl.snapkv_inputs(cfg, dev)
        q, k, v = self.inp["q"], self.inp["k"], self.inp["v"]
        U, N, D = cfg.U, cfg.N, cfg.D
        self.lse = torch.empty((cfg.L, cfg.Hq, cfg.W), dtype=torch.float32, device=dev)
        self.scores = torch.empty((U, N), dtype=torch.float32, device=dev)
        self.kept = torch.empty((U, cfg.k), dtype=torch.int32, device=dev)
        self.dk = torch.empty((U, cfg.k, D), dtype=k.dtype, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.k3, self.v3 = k.view(U, N, D), v.view(U, N, D)
        self.ws = kv.score_window(q, k, None, lse_out=self.lse)
        self.sel_ws = kv.select(self.scores, self.kept, k_total=cfg.k, n_sink=cfg.n_sink,
                                n_recent=cfg.n_recent, pool=cfg.pool, pool_k=cfg.pool_k)
        self.tokens = cfg.L * cfg.Hkv * N

    def step(self, ev, stream, it):
        kv, cfg, q, k = self.kv, self.cfg, self.inp["q"], self.inp["k"]
        ev[0].record(stream)
        kv.score_window(q, k, None, lse_out=self.lse, workspace=self.ws)
        ev[1].record(stream)
        kv.score_window(q, k, self.scores, lse_in=self.lse)
        ev[2].record(stream)
        kv.select(self.scores, self.kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  pool=cfg.pool, pool_k=cfg.pool_k, workspace=self.sel_ws)
        ev[3].record(stream)
        kv.gather_rerope(self.k3, self.v3, self.kept, self.dk, self.dv, bt=1, D=cfg.D, src_rows=cfg.N,
                         src_unit_stride=cfg.N * cfg.D)
        ev[4].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        kb = cfg.L * cfg.Hkv * cfg.N * cfg.D * 2
        qb = cfg.L * cfg.Hq * cfg.W * cfg.D * 2
        lb = cfg.L * cfg.Hq * cfg.W * 4
        sb = cfg.U * cfg.N * 4
        kept_b = cfg.U * cfg.k * 4
        gb = 2 * 2 * cfg.U * cfg.k * cfg.D * 2
        return {"lse": kb + qb + lb, "score": kb + qb + lb + sb, "select": sb + kept_b, "gather": kept_b + gb}

    def mfma_flops(self):
        cfg = self.cfg
        f = 2 * cfg.G * cfg.W * cfg.N * cfg.D * cfg.U      # q . k for every (row, key) of every unit
        return {"lse": f, "score": f}

    def cpu_baseline(self, seconds):
        """Whole units in a seeded order: window scores with the oracle's own
        LSE, max-pool, top-k, gather."""
        import numpy as np
        from oracle import materialise as om
        from oracle import numerics
        from oracle import score as osc
        from oracle import select as osel
        cfg, inp = self.cfg, self.inp
        clock = OracleTimer(seconds)
        done = 0
        for u in np.random.default_rng(cfg.seed).permutation(cfg.U):
            l, g = divmod(int(u), cfg.Hkv)
            q = _np64(inp["q"][l:l + 1, g * cfg.G:(g + 1) * cfg.G])
            k = _np64(inp["k"][l:l + 1, g:g + 1])
            v = _np64(inp["v"][l, g])
            a, _ = clock.run(osc.window_scores, q, k)
            pooled = clock.run(osc.pool1d, a[0, 0], cfg.pool, cfg.pool_k)
            kept, _ = clock.run(osel.select_topk, numerics.round_to_f32(pooled), cfg.k, cfg.n_sink, cfg.n_recent)
            clock.run(om.gather_view, k[0, 0], v, kept, 1)
            done += 1
            if clock.spent():
                break
        return clock.result(done * cfg.N, "%d of %d (layer, KV head) units in seeded order, full N=%d each: "
                            "window scores (LSE computed), max-pool, top-k, gather" % (done, cfg.U, cfg.N))

    def config(self):
        cfg = self.cfg
        return {"workload": "snapkv-h2o token scoring: 36 layers x 8 KV heads (32 query heads) x "
                            "32768 tokens x D128 bf16, window 64, max-pool 7, top 8192 per (layer, KV "
                            "head) with 4 sink + 256 recent, gather K+V",
                "units": cfg.U, "tokens_per_unit": cfg.N, "budget": cfg.k}

    def extra(self):
        return {}


class IntentKV:
    """Session-memory scoring over a paged pool: one turn's memory update,
    memory-attention rule scores summed over every layer and head, a global
    top-8192 (dead slots excluded), the alias-aware free list of the step
    (the 4-token sink prefix as the radix-protected prefix), and the slot-map redirect
    with sentinel rows.  The slot map is reset from the original before each
    step (a 256 KiB copy outside the stage events) so every step does the
    same work."""
    stages = ["update", "score", "select", "free", "redirect"]
    dominant = ("score", [("memory_logits_mfma_kernel", "k_memory.hip"), ("memory_lse_kernel", "k_memory.hip"),
                          ("memory_rule_kernel", "k_memory.hip"), ("memory_layer_sum_kernel", "k_memory.hip")])
    score_stage = "score"
    materialise_stages = ["select", "free", "redirect"]
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.kv, self.cfg = kv, wl.CONFIGS["intentkv"]
        cfg = self.cfg
        self.inp = wl.intentkv_inputs(cfg, dev)
        L, Hq, D, N = cfg.L, cfg.Hq, cfg.D, cfg.N
        self.m = torch.zeros((L, Hq, D), dtype=torch.float32, device=dev)
        self.rule = torch.empty(N, dtype=torch.float32, device=dev)
        self.kept = torch.empty((1, cfg.k), dtype=torch.int32, device=dev)
        self.mask = torch.empty((1, N), dtype=torch.uint8, device=dev)
        self.sm = self.inp["slot_map"].clone()
        self.kflat = self.inp["k_pool"].view(L, -1, cfg.Hkv, D)
        self.vflat = self.inp["v_pool"].view(L, -1, cfg.Hkv, D)
        kv.memory_update(self.inp["turns"][0], self.m, decay=cfg.decay)
        self.ws = kv.score_memory(self.m, self.inp["k_pool"], self.inp["page_table"], N, self.rule,
                                  page_size=cfg.page_size, slot_map=self.sm, dead_slot=self.inp["dead_slot"],
                                  n_sink=cfg.n_sink, n_recent=cfg.n_recent)
        self.sel_ws = kv.select(self.rule[None], self.kept, k_total=cfg.k, n_sink=cfg.n_sink,
                                n_recent=cfg.n_recent, keep_mask=self.mask, slot_map=self.sm,
                                dead_slot=self.inp["dead_slot"])
        self.freed = torch.empty(N, dtype=torch.int32, device=dev)
        self.n_freed = torch.empty(1, dtype=torch.int32, device=dev)
        self.n_slots = (self.inp["page_table"].numel() + 1) * cfg.page_size   # pages + the dead page
        self.free_ws = kv.free_list(self.sm, self.mask[0], self.inp["dead_slot"], self.freed, self.n_freed,
                                    n_slots=self.n_slots, protected_len=0)
        self.tokens = cfg.L * cfg.Hkv * N

    def step(self, ev, stream, it):
        kv, cfg, inp = self.kv, self.cfg, self.inp
        self.sm.copy_(inp["slot_map"])
        ev[0].record(stream)
        kv.memory_update(inp["turns"][it % cfg.turns], self.m, decay=cfg.decay)
        ev[1].record(stream)
        kv.score_memory(self.m, inp["k_pool"], inp["page_table"], cfg.N, self.rule, page_size=cfg.page_size,
                        slot_map=self.sm, dead_slot=inp["dead_slot"], n_sink=cfg.n_sink,
                        n_recent=cfg.n_recent, workspace=self.ws)
        ev[2].record(stream)
        kv.select(self.rule[None], self.kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  keep_mask=self.mask, slot_map=self.sm, dead_slot=inp["dead_slot"], workspace=self.sel_ws)
        ev[3].record(stream)
        kv.free_list(self.sm, self.mask[0], inp["dead_slot"], self.freed, self.n_freed, n_slots=self.n_slots,
                     protected_len=cfg.n_sink, workspace=self.free_ws)
        ev[4].record(stream)
        kv.redirect(self.sm, self.mask[0], inp["dead_slot"], k_pool=self.kflat, v_pool=self.vflat)
        ev[5].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        N, L, Hq, Hkv, D = cfg.N, cfg.L, cfg.Hq, cfg.Hkv, cfg.D
        mb = L * Hq * D * 4
        return {"update": L * Hq * cfg.W * D * 2 + 2 * mb,
                "score": L * N * Hkv * D * 2 + mb + 4 * N + 4 * (N // cfg.page_size) + 4 * N,
                "select": 4 * N + 4 * N + N + 4 * cfg.k,
                "free": 2 * (4 * N + N) + 4 * N,
                "redirect": 2 * 4 * N + N + 2 * L * Hkv * D * 2}

    def cpu_baseline(self, seconds):
        """One whole step on the oracle (it fits the budget): the memory update
        with one turn, the rule score over all 36 layers (the per-layer sums
        added in layer order), the global top-k with dead slots excluded, the
        free list and the redirect."""
        import numpy as np
        from oracle import materialise as om
        from oracle import numerics
        from oracle import score as osc
        from oracle import select as osel
        cfg, inp = self.cfg, self.inp
        L, N, ps = cfg.L, cfg.N, cfg.page_size
        clock = OracleTimer(seconds)
        turn = _np64(inp["turns"][0])
        pool32 = inp["k_pool"].float().cpu().numpy()                  # [L][P][ps][Hkv][D], float32 (exact)
        pt = inp["page_table"].cpu().numpy().astype(np.int64)
        sm = inp["slot_map"].cpu().numpy().astype(np.int64)
        dead = int(inp["dead_slot"])
        m = clock.run(osc.memory_update, np.zeros((L, cfg.Hq, cfg.D)), turn, decay=cfg.decay)
        m32 = numerics.round_to_f32(m)
        rule = np.zeros(N)
        layers = 0
        for l in range(L):
            rule += clock.run(osc.memory_scores, m32[l:l + 1], pool32[l:l + 1], pt, ps, N, slot_map=sm,
                              dead_slot=dead, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
            layers += 1
        alive = sm != dead
        _, mask = clock.run(osel.select_topk, numerics.round_to_f32(rule), cfg.k, cfg.n_sink, cfg.n_recent, alive)
        clock.run(om.free_list, sm, mask, dead, protected_len=cfg.n_sink)
        clock.run(om.redirect, sm, mask, dead)
        return clock.result(layers * cfg.Hkv * N, "one whole step (%d of %d layers): memory update, rule scores, "
                            "global top-%d, free list, redirect" % (layers, L, cfg.k))

    def config(self):
        cfg = self.cfg
        return {"workload": "intentkv session-memory scoring: 36 layers x 8 KV heads (32 query heads) x "
                            "65536 tokens x D128 bf16 in 16-token pages, memory update over a 64-query "
                            "turn (decay 0.9), global top 8192 with 4 sink + 64 recent, alias-aware free list, "
                            "dead-slot redirect",
                "units": 1, "tokens_per_unit": cfg.N, "budget": cfg.k, "protected_prefix": cfg.n_sink}

    def extra(self):
        return {}


class KVMem1M:
    """Block retrieval over a 1M-token workspace: query reduction and Mean-K
    block scores, per-unit top-2048 blocks, raw-K gather re-RoPEd to
    contiguous positions with V copied."""
    stages = ["score", "select", "gather"]
    dominant = ("gather", [("gather_blocks_kernel", "k_gather.hip")])
    score_stage = "score"
    materialise_stages = ["select", "gather"]
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.torch, self.kv, self.cfg = torch, kv, wl.CONFIGS["kvmem1m"]
        cfg = self.cfg
        self.mu, w, _ = wl.kvmem_index(cfg, dev)
        self.q = wl.kvmem_queries(cfg, dev, w, 0)[None]
        self.raw_k, self.raw_v, self.offs = wl.kvmem_raw_store(cfg, dev)
        U, NB, k, D, bt = cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt
        self.scores = torch.empty((1, U, NB), dtype=torch.float32, device=dev)
        self.qbar = torch.empty((1, cfg.L, cfg.Hkv, D), dtype=torch.float32, device=dev)
        self.kept = torch.empty((U, k), dtype=torch.int32, device=dev)
        self.vk = torch.empty((U, k * bt, D), dtype=torch.bfloat16, device=dev)
        self.vv = torch.empty_like(self.vk)
        self.ws = kv.score_block(self.q, self.mu, self.scores, n_kv_heads=cfg.Hkv, qbar=self.qbar)
        self.sel_ws = kv.select(self.scores[0], self.kept, k_total=k, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
        self.tokens = U * NB * bt

    def step(self, ev, stream, it):
        kv, cfg = self.kv, self.cfg
        ev[0].record(stream)
        kv.score_block(self.q, self.mu, self.scores, n_kv_heads=cfg.Hkv, qbar=self.qbar, workspace=self.ws)
        ev[1].record(stream)
        kv.select(self.scores[0], self.kept, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                  workspace=self.sel_ws)
        ev[2].record(stream)
        kv.gather_rerope(self.raw_k, self.raw_v, self.kept, self.vk, self.vv, bt=cfg.bt, D=cfg.D,
                         src_rows=cfg.N * cfg.bt, src_offsets=self.offs, rope="raw", theta=cfg.theta)
        ev[3].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        U, NB, k, D, bt = cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt
        sb = U * NB * 4
        return {"score": cfg.L * cfg.Hq * cfg.W * D * 2 + U * NB * D * 2 + sb,
                "select": sb + U * k * 4,
                "gather": U * k * 4 + 2 * 2 * U * k * bt * D * 2}

    def cpu_baseline(self, seconds):
        """Whole units in a seeded order: query reduction, block scores over all
        32768 blocks, top-2048, raw-K gather re-RoPEd at theta 1e6 with V."""
        import numpy as np
        from oracle import materialise as om
        from oracle import numerics
        from oracle import score as osc
        from oracle import select as osel
        cfg = self.cfg
        clock = OracleTimer(seconds)
        done = 0
        for u in np.random.default_rng(cfg.seed).permutation(cfg.U):
            l, g = divmod(int(u), cfg.Hkv)
            q = _np64(self.q[:, l:l + 1, g * cfg.G:(g + 1) * cfg.G])
            mu = _np64(self.mu[l:l + 1, g:g + 1])
            qb = clock.run(osc.query_reduce, q, 1)
            sc = clock.run(osc.block_scores, qb, mu)[0, 0, 0]
            kept, _ = clock.run(osel.select_topk, numerics.round_to_f32(sc), cfg.k, cfg.n_sink, cfg.n_recent)
            buf = l % cfg.raw_layers
            sel = self.torch.from_numpy(kept).to(self.raw_k.device)
            rk = _np64(self.raw_k[buf, g][sel]).reshape(-1, cfg.D)         # the kept blocks, in kept order
            rv = _np64(self.raw_v[buf, g][sel]).reshape(-1, cfg.D)
            clock.run(om.gather_view, rk, rv, np.arange(len(kept)), cfg.bt, rope="raw", theta=cfg.theta)
            done += 1
            if clock.spent():
                break
        return clock.result(done * cfg.N * cfg.bt, "%d of %d (layer, KV head) units in seeded order, all %d "
                            "blocks each: query reduction, block scores, top-%d, raw-K gather with re-RoPE"
                            % (done, cfg.U, cfg.N, cfg.k))

    def config(self):
        cfg = self.cfg
        return {"workload": "kvmem 1M-token block retrieval: 64 layers x 8 KV heads (64 query heads), "
                            "32768 32-token blocks per unit, fp16 Mean-K, 512-token query, top 2048 blocks "
                            "(block 0 + last 4 forced), raw-K gather re-RoPEd at theta 1e6, V copied",
                "units": cfg.U, "blocks_per_unit": cfg.N, "budget_blocks": cfg.k}

    def extra(self):
        return {}


class KVMem10M:
    """Scale-out block retrieval: a 10M-token Mean-K index scored in
    65536-block tiles for 4 sessions with a running tiled top-4096, then the
    in-place incremental update of each session's 4096-page view (the
    previous view shares about half its blocks with the new selection;
    misses and moved hits are re-RoPEd from the raw store at their new
    positions, V is copied for misses only).
    Tiles after the first are scored in the packed form: only the blocks
    above their running set's smallest score are written (the selection's
    admission threshold), with a bit mask.  The previous-view lists are
    inputs, so every step does the same work."""
    stages = ["tiles", "update"]
    dominant = ("update", [("incremental_data_kernel", "k_incremental.hip"),
                           ("incremental_plan_kernel", "k_incremental.hip")])
    score_stage = "tiles"
    materialise_stages = ["update"]
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        import numpy as np
        self.torch, self.kv, self.cfg = torch, kv, wl.CONFIGS["kvmem10m"]
        cfg = self.cfg
        S, U, NB, k, D, bt, tile = cfg.S, cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt, cfg.tile
        room = k - cfg.n_sink - cfg.n_recent
        self.mu, w, planted = wl.kvmem_index(cfg, dev, n_dirs=S, planted=(room, 10.0))
        self.qs = torch.stack([wl.kvmem_queries(cfg, dev, w, s) for s in range(S)])
        SU = S * U
        self.qbar = torch.empty((S, cfg.L, cfg.Hkv, D), dtype=torch.float32, device=dev)
        self.cs = torch.empty((SU, k), dtype=torch.float32, device=dev)
        self.ci = torch.empty((SU, k), dtype=torch.int32, device=dev)
        self.cc = torch.zeros(SU, dtype=torch.int32, device=dev)
        self.kept = torch.empty((SU, k), dtype=torch.int32, device=dev)
        self.tile_out = torch.empty((S, U, tile), dtype=torch.float32, device=dev)
        self.mask = torch.empty((SU * ((tile + 63) // 64),), dtype=torch.int64, device=dev)
        self.admit = torch.empty((SU,), dtype=torch.float32, device=dev)
        self.admitted = None
        self.raw_k = torch.empty((cfg.Hkv, NB, bt, D), dtype=torch.bfloat16, device=dev)
        self.raw_v = torch.empty_like(self.raw_k)
        gen = torch.Generator(device=dev).manual_seed(cfg.seed + 77)
        for h in range(cfg.Hkv):
            self.raw_k[h].normal_(generator=gen)
            self.raw_v[h].normal_(generator=gen)
        self.offs = torch.tensor([((i % U) % cfg.Hkv) * NB * bt * D for i in range(SU)], dtype=torch.int64,
                                 device=dev)
        rng = np.random.default_rng(cfg.seed)
        prev_idx = np.empty((SU, k), np.int32)
        prev_page = np.empty((SU, k), np.int32)
        planted_h = planted.cpu().numpy()
        for i in range(SU):
            s, u = divmod(i, U)
            l, g = divmod(u, cfg.Hkv)
            inside = rng.choice(planted_h[s, l, g], k // 2, replace=False)
            taken = np.zeros(NB, bool)
            taken[planted_h[s, l, g]] = True
            draw = np.unique(rng.integers(0, NB, 3 * k))
            draw = draw[~taken[draw]]
            outside = rng.choice(draw, k - k // 2, replace=False)
            prev_idx[i] = np.sort(np.concatenate([inside, outside]))
            prev_page[i] = rng.permutation(k)
        self.prev_idx_h = prev_idx
        self.prev_idx = torch.from_numpy(prev_idx).to(dev)
        self.prev_page = torch.from_numpy(prev_page).to(dev)
        self.pool_k = torch.full((SU, k, bt, D), 0.5, dtype=torch.bfloat16, device=dev)
        self.pool_v = torch.full((SU, k, bt, D), -0.25, dtype=torch.bfloat16, device=dev)
        self.pt = torch.empty((SU, k), dtype=torch.int32, device=dev)
        self.nm = torch.empty(SU, dtype=torch.int32, device=dev)
        self.tokens = S * U * NB * bt
        self.ws = None
        self.sel_ws = None
        self.inc_ws = None

    def _tiles(self, count=False):
        """The tile loop; with count, the admitted columns of every packed
        tile (an untimed pass for the algorithmic bytes)."""
        import numpy as np
        kv, cfg = self.kv, self.cfg
        S, U, NB, k, tile = cfg.S, cfg.U, cfg.N, cfg.k, cfg.tile
        SU = S * U
        admitted = []
        self.cc.zero_()
        for b in range(0, NB, tile):
            n = min(tile, NB - b)
            out = self.tile_out.view(-1)[: SU * n]
            packed = b > 0
            mask = self.mask[: SU * ((n + 63) // 64)] if packed else None
            self.ws = kv.score_block(self.qs if b == 0 else None, self.mu, out.view(S, U, n), n_kv_heads=cfg.Hkv,
                                     n_begin=b, n_count=n, qbar=self.qbar, qbar_valid=b > 0,
                                     admit=self.admit.view(S, U) if packed else None, tile_mask=mask,
                                     workspace=self.ws)
            self.sel_ws = kv.select(out.view(SU, n), self.kept, k_total=k, n_sink=cfg.n_sink,
                                    n_recent=cfg.n_recent, n_total=NB, base=b, cand_score=self.cs,
                                    cand_idx=self.ci, cand_count=self.cc, finalize=b + n == NB,
                                    tile_mask=None if mask is None else mask.view(SU, -1),
                                    admit=self.admit if b + n < NB else None, workspace=self.sel_ws)
            if count and packed:
                admitted.append(int(np.unpackbits(mask.cpu().numpy().view(np.uint8)).sum()))
        return admitted

    def step(self, ev, stream, it):
        kv, cfg, NB = self.kv, self.cfg, self.cfg.N
        ev[0].record(stream)
        self._tiles()
        ev[1].record(stream)
        self.inc_ws = kv.gather_incremental(self.raw_k, self.raw_v, self.kept, self.prev_idx, self.prev_page,
                                            self.pool_k, self.pool_v, self.pt, self.nm, bt=cfg.bt, D=cfg.D,
                                            src_rows=NB * cfg.bt, src_offsets=self.offs, rope="raw",
                                            theta=cfg.theta, hit_raw=True, workspace=self.inc_ws)
        ev[2].record(stream)

    def _moves(self):
        import numpy as np
        new = self.kept.cpu().numpy()
        misses = int(self.nm.sum())
        moved = 0
        for i in range(new.shape[0]):
            common, ia, ib = np.intersect1d(self.prev_idx_h[i], new[i], assume_unique=True, return_indices=True)
            moved += int(np.count_nonzero(ia != ib))
        return misses, moved

    def algo_bytes(self):
        cfg = self.cfg
        S, U, NB, k, D, bt, tile = cfg.S, cfg.U, cfg.N, cfg.k, cfg.D, cfg.bt, cfg.tile
        SU = S * U
        misses, moved = self._moves()
        if self.admitted is None:
            self.admitted = self._tiles(count=True)
        n_tiles = (NB + tile - 1) // tile
        blk = bt * D * 2
        # index once, queries once; the first tile's scores written and read;
        # later tiles: admitted scores written and read, mask words written
        # and read; the running candidates (score + index) read and written
        # by every select call
        scores = 2 * SU * min(tile, NB) * 4 + 2 * sum(self.admitted) * 4 + 2 * SU * ((NB - tile + 63) // 64) * 8
        cands = n_tiles * 2 * SU * k * 8
        return {"tiles": U * NB * D * 2 + S * cfg.L * cfg.Hq * cfg.W * D * 2 + scores + cands,
                "update": misses * 2 * 2 * blk + moved * 2 * blk + 3 * SU * k * 4}

    def cpu_baseline(self, seconds):
        """Whole (session, unit) views in a seeded order: the query reduction,
        block scores over all 312500 blocks, the top-4096 (the tiled selection
        is defined equal to the untiled one, so the oracle selects once), and
        the incremental update of that view (misses and moved hits re-RoPEd
        from raw K at their new positions)."""
        import numpy as np
        from oracle import materialise as om
        from oracle import numerics
        from oracle import score as osc
        from oracle import select as osel
        torch, cfg = self.torch, self.cfg
        S, U, NB, k, bt, D = cfg.S, cfg.U, cfg.N, cfg.k, cfg.bt, cfg.D
        clock = OracleTimer(seconds)
        done = 0
        t_update = 0.0
        prev_page = self.prev_page.cpu().numpy()
        for i in np.random.default_rng(cfg.seed).permutation(S * U):
            s, u = divmod(int(i), U)
            l, g = divmod(u, cfg.Hkv)
            q = _np64(self.qs[s:s + 1, l:l + 1, g * cfg.G:(g + 1) * cfg.G])
            mu = _np64(self.mu[l:l + 1, g:g + 1])
            qb = clock.run(osc.query_reduce, q, 1)
            sc = clock.run(osc.block_scores, qb, mu)[0, 0, 0]
            del mu
            kept, _ = clock.run(osel.select_topk, numerics.round_to_f32(sc), k, cfg.n_sink, cfg.n_recent)
            # the raw blocks this update reads, renumbered by rank (order kept)
            need = np.union1d(self.prev_idx_h[i], kept)
            sel = torch.from_numpy(need).to(self.raw_k.device)
            rk, rv = _np64(self.raw_k[g][sel]), _np64(self.raw_v[g][sel])
            pk, pv = _np64(self.pool_k[i]), _np64(self.pool_v[i])
            b0 = clock.busy
            clock.run(om.incremental_view, np.searchsorted(need, self.prev_idx_h[i]), prev_page[i],
                      np.searchsorted(need, kept), pk, pv, rk, rv, bt, theta=cfg.theta, hits="raw")
            t_update += clock.busy - b0
            done += 1
            if clock.spent():
                break
        return clock.result(done * NB * bt, "%d of %d (session, layer, KV head) views in seeded order, all %d "
                            "blocks each: query reduction, block scores, top-%d, incremental view update "
                            "(%.1f s of it the update)" % (done, S * U, NB, k, t_update))

    def config(self):
        cfg = self.cfg
        return {"workload": "kvmem 10M-token scale-out retrieval: 64 layers x 8 KV heads, 312500 32-token "
                            "blocks per unit scored in 65536-block tiles for 4 sessions, tiled top 4096, "
                            "in-place incremental update of 4096-page views with about half the blocks reused "
                            "(misses and moved hits re-RoPEd from raw K)",
                "units": cfg.U, "sessions": cfg.S, "blocks_per_unit": cfg.N, "budget_blocks": cfg.k}

    def extra(self):
        misses, moved = self._moves()
        return {"update_misses": misses, "update_moved_hits": moved,
                "admitted_per_packed_tile": self.admitted}


class MeanK1M:
    """Building the whole Mean-K index of the 1M-token workspace: the fp16
    mean of every 32-token block of raw keys, for 64 layers x 8 KV heads x
    32768 blocks (the layers read 8 aliased raw buffers, as in kvmem1m)."""
    stages = ["index"]
    dominant = ("index", [("mean_k_kernel", "k_index.hip")])
    score_stage = "index"
    materialise_stages = []
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.kv, self.cfg = kv, wl.CONFIGS["kvmem1m"]
        cfg = self.cfg
        self.raw_k, _, self.offs = wl.kvmem_raw_store(cfg, dev)
        self.mu = torch.empty((cfg.U, cfg.N, cfg.D), dtype=torch.float16, device=dev)
        self.tokens = cfg.U * cfg.N * cfg.bt

    def step(self, ev, stream, it):
        cfg = self.cfg
        ev[0].record(stream)
        self.kv.build_index(self.raw_k, self.mu, bt=cfg.bt, D=cfg.D, src_rows=cfg.N * cfg.bt, src_offsets=self.offs)
        ev[1].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        return {"index": cfg.U * cfg.N * cfg.bt * cfg.D * 2 + cfg.U * cfg.N * cfg.D * 2}

    def cpu_baseline(self, seconds):
        """Whole units in a seeded order: the float64 mean of every 32-row
        block of the unit's raw keys, rounded once to fp16."""
        import numpy as np
        from oracle import score as osc
        cfg = self.cfg
        clock = OracleTimer(seconds)
        done = 0
        raw = self.raw_k.view(-1, cfg.N * cfg.bt, cfg.D)
        for u in np.random.default_rng(cfg.seed).permutation(cfg.U):
            l, g = divmod(int(u), cfg.Hkv)
            x = _np64(raw[(l % cfg.raw_layers) * cfg.Hkv + g])
            clock.run(osc.mean_k_index, x, cfg.bt)
            del x
            done += 1
            if clock.spent():
                break
        return clock.result(done * cfg.N * cfg.bt, "%d of %d (layer, KV head) units in seeded order, all %d "
                            "blocks of %d raw rows each" % (done, cfg.U, cfg.N, cfg.bt))

    def config(self):
        cfg = self.cfg
        return {"workload": "kvmem Mean-K index build over the 1M-token workspace: 64 layers x 8 KV heads x "
                            "32768 blocks of 32 raw bf16 keys (D128) -> fp16 block means",
                "units": cfg.U, "blocks_per_unit": cfg.N, "block_tokens": cfg.bt}

    def extra(self):
        return {}


class ActKVCompact:
    """One ActKV compression step with Table 1's shape, for 64 requests that
    just left an action region (6144 positions each, 16-slot blocks, 36
    layers of 8 KV heads, D 128, bf16): the LRFU keep score from the action
    scorer's running means (lambda 0.5, top-p 0.9), eviction to 4096 kept
    entries by keep score (4 sink + 64 recent forced), and the in-place tail
    compaction of K and V.  The keep scores start at the policy's fixed
    point for this state (2 * score on hits, smaller tail-weighted values
    elsewhere), so every step computes the same keep mask and repeats the
    same moves."""
    stages = ["keep_score", "select", "compact"]
    dominant = ("compact", [("compact_copy_kernel", "k_compact.hip"), ("compact_plan_kernel", "k_compact.hip")])
    score_stage = "keep_score"
    materialise_stages = ["select", "compact"]
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.kv, self.cfg = kv, wl.CONFIGS["actkv"]
        cfg = self.cfg
        self.inp = wl.actkv_inputs(cfg, dev)
        R, N, bs = cfg.S, cfg.N, cfg.page_size
        Y = self.inp["block_table"].shape[1]
        self.state = wl.actkv_state(cfg, dev)
        self.n_len = torch.full((R,), N, dtype=torch.int32, device=dev)
        # the fixed point of KS <- 0.5 KS + hit * score: 2 * score on hits;
        # the other entries sit below every hit, ordered toward the tail
        ks = torch.zeros((R, N), dtype=torch.float32, device=dev)
        hit = torch.empty((R, N), dtype=torch.uint8, device=dev)
        kv.keep_score(self.state, ks, self.n_len, lam=0.0, top_p=0.9, hit=hit)
        floor = torch.where(hit.bool(), ks, torch.full_like(ks, float("inf"))).amin(dim=1, keepdim=True)
        ramp = torch.linspace(0.1, 0.4, N, device=dev)[None]
        self.ks = torch.where(hit.bool(), 2.0 * ks, floor * ramp).contiguous()
        self.hits = int(hit.sum())
        self.kept_idx = torch.empty((R, cfg.k), dtype=torch.int32, device=dev)
        self.keep = torch.empty((R, N), dtype=torch.uint8, device=dev)
        self.slot_pos = torch.empty((R, Y * bs), dtype=torch.int32, device=dev)
        self.freed = torch.empty((R, Y), dtype=torch.int32, device=dev)
        self.n_freed = torch.empty(R, dtype=torch.int32, device=dev)
        self.ws_keep = self.ws_sel = self.ws = None
        self.tokens = R * cfg.N * cfg.L * cfg.Hkv
        self.pairs = None
        self.torch = torch

    def step(self, ev, stream, it):
        inp, cfg, kv = self.inp, self.cfg, self.kv
        ev[0].record(stream)
        self.ws_keep = kv.keep_score(self.state, self.ks, self.n_len, lam=cfg.decay, top_p=0.9,
                                     workspace=self.ws_keep)
        ev[1].record(stream)
        self.ws_sel = kv.select(self.ks, self.kept_idx, k_total=cfg.k, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                                keep_mask=self.keep, workspace=self.ws_sel)
        ev[2].record(stream)
        self.ws = kv.compact(self.keep, inp["block_table"], inp["k_pool"], inp["v_pool"], self.slot_pos,
                             self.freed, self.n_freed, block_size=cfg.page_size, workspace=self.ws)
        ev[3].record(stream)

    def _moved(self):
        if self.pairs is None:
            cfg, bs = self.cfg, self.cfg.page_size
            Y = self.inp["block_table"].shape[1]
            keep = self.keep.bool()
            X = (keep.sum(dim=1) + bs - 1) // bs
            t0 = (Y - X) * bs
            pos = self.torch.arange(cfg.N, device=keep.device)[None]
            self.pairs = int((keep & (pos < t0[:, None])).sum())      # one (source, destination) copy each
        return self.pairs

    def algo_bytes(self):
        cfg = self.cfg
        R, N, bs = cfg.S, cfg.N, cfg.page_size
        Y = self.inp["block_table"].shape[1]
        row = cfg.Hkv * cfg.D * 2
        moves = self._moved() * cfg.L * 2 * 2 * row                  # K and V, read and written
        return {"keep_score": cfg.L * R * cfg.Hkv * N * 4 + R * N * 4 * 4,   # state; scores out, in; KS r/w
                "select": R * N * 4 + R * N + R * cfg.k * 4,
                "compact": moves + R * N + R * Y * 4 + R * Y * bs * 4 + R * Y * 4}

    def config(self):
        cfg = self.cfg
        return {"workload": "actkv compression step: LRFU keep score (lambda 0.5, top-p 0.9) from 36 layers x "
                            "8 KV heads of running means, eviction to 4096 of 6144 positions by keep score, "
                            "in-place tail compaction of 64 requests' 16-slot bf16 paged K/V (D128)",
                "requests": cfg.S, "positions": cfg.N, "kept": cfg.k, "block_size": cfg.page_size,
                "lambda": cfg.decay, "top_p": 0.9}

    def extra(self):
        return {"moved_entries": self._moved(), "top_p_hits": self.hits}


class ActKVDecode:
    """One decode token of ActKV's recovery-based action scorer for 64
    requests at 6144 positions (36 layers, 8 KV / 32 query heads, D 128,
    bf16 paged K in 16-slot blocks): logits recomputed from the paged keys,
    probabilities recovered with the attention pass's LSE, the maximum over
    each GQA group folded into the running mean (5 tokens already in it).
    Repeating the step with the same token count repeats the same work."""
    stages = ["decode"]
    dominant = ("decode", [("decode_score_kernel", "k_decode.hip")])
    score_stage = "decode"
    materialise_stages = []
    dtype = "bf16"

    def __init__(self, torch, kv, wl, dev):
        self.kv, self.cfg = kv, wl.CONFIGS["actkv"]
        self.inp = wl.actkv_decode_inputs(self.cfg, dev)
        self.state = wl.actkv_state(self.cfg, dev)
        cfg = self.cfg
        self.tokens = cfg.S * cfg.N * cfg.L * cfg.Hkv

    def step(self, ev, stream, it):
        inp = self.inp
        ev[0].record(stream)
        self.kv.decode_score(inp["q"], inp["lse"], inp["k_pool"], inp["block_table"], inp["n_ctx"], inp["n_seen"],
                             self.state)
        ev[1].record(stream)

    def algo_bytes(self):
        cfg = self.cfg
        R, N = cfg.S, cfg.N
        keys = cfg.L * R * N * cfg.Hkv * cfg.D * 2
        state = 2 * cfg.L * R * cfg.Hkv * N * 4                        # read and written (mid-region)
        small = cfg.L * R * cfg.Hq * (cfg.D * 2 + 4) + R * (N // cfg.page_size) * 4
        return {"decode": keys + state + small}

    def config(self):
        cfg = self.cfg
        return {"workload": "actkv decode-streaming recovery scorer: one action token of 64 requests x 6144 "
                            "positions, 36 layers x 8 KV / 32 query heads x D128 bf16 paged K (16-slot blocks), "
                            "LSE from the attention pass, max over the GQA group, running mean",
                "requests": cfg.S, "positions": cfg.N, "block_size": cfg.page_size, "tokens_in_mean": cfg.turns}

    def extra(self):
        return {}


WORKLOADS = {"tiny": Tiny, "snapkv": SnapKV, "intentkv": IntentKV, "kvmem1m": KVMem1M, "kvmem10m": KVMem10M,
             "meank1m": MeanK1M, "actkv": ActKVCompact, "actkv_decode": ActKVDecode}


def main():
    args = _args()
    if args.gpus != 1:
        print("bench.py measures one GPU only; a run on several GPUs is not built "
              "(the (layer, KV head) units would shard across GPUs without any exchange)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, args.command, args.workload)
        return
    if args.copy_calib:
        copy_calibration()
        return
    import torch
    import selection_score_amd as kv
    from selection_score_amd import workloads as wl

    dev = torch.device("cuda:0")
    wk = WORKLOADS[args.workload](torch, kv, wl, dev)
    stream = torch.cuda.current_stream()
    copy_gbps = copy_reference(stream)
    n_ev = len(wk.stages) + 1
    flush = getattr(wk, "flush", False)
    pre = getattr(wk, "pre_step", lambda: None)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    warm = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for i in range(args.warmup):
        if flush:
            pre()
        wk.step(warm, stream, i)
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        if flush:
            pre()
        wk.step(evs[i], stream, args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    per = {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(wk.stages)}
    spans = [e[0].elapsed_time(e[-1]) for e in evs]         # each step's own span
    if flush:
        # latency: each step's own span, the cache flush before it excluded
        ms_step = sum(spans) / args.steps
    else:
        ms_step = t_start.elapsed_time(t_end) / args.steps
    stage = {n: sum(t) / len(t) for n, t in per.items()}
    algo = wk.algo_bytes()
    step_bytes = sum(algo.values())
    # the longest kernel of the step: one library call per step, so its stage
    # time is one launch (plus the short companion launches of the same call)
    dom_stage, dom_kernels = wk.dominant
    achieved = algo[dom_stage] / (stage[dom_stage] * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": wk.tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wk.dtype,
        "data": "synthetic",
        "config": wk.config(),
        "stages_ms": stage,
        "step_ms_median": statistics.median(spans),
        "step_ms_min": min(spans),
        "stages_ms_median": {n: statistics.median(t) for n, t in per.items()},
        "stages_ms_min": {n: min(t) for n, t in per.items()},
        "stage_gbps": {n: algo[n] / (stage[n] * 1e-3) / 1e9 for n in wk.stages},
        "score_pass_tokens_per_s": wk.tokens / (stage[wk.score_stage] * 1e-3),
        "step_hbm_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "select_gather_ms": sum(stage[n] for n in wk.materialise_stages),
        "copy_reference_gbps": copy_gbps,
        "roofline": {"bound": "hbm", "kernel": dom_kernels[0][0], "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": _kernels_traffic(dom_kernels, args.workload), "algorithmic_bytes": algo[dom_stage],
                     "launch_ms": stage[dom_stage], "stage": dom_stage,
                     "companions": [k for k, _ in dom_kernels[1:]]},
        "cpu_baseline": None,
    }
    flops = getattr(wk, "mfma_flops", lambda: {})()
    if flops:
        # the matrix-core side of the co-bound window passes: dense bf16 MFMA
        # work per launch over the stage time, against the dense bf16 peak
        out["mfma"] = {n: {"achieved": f / (stage[n] * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": f / (stage[n] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                           "flops": f} for n, f in flops.items()}
    out.update(wk.extra())
    if not args.no_cpu_baseline and hasattr(wk, "cpu_baseline"):
        out["cpu_baseline"] = wk.cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)

if __name__ == "__main__":
    main()
