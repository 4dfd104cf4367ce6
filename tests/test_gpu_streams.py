"""Calls from several host threads, each on its own stream with its own
workspace, run concurrently and give the same results as one after another.
The library keeps no state between calls except a per-device check of the
architecture and a per-thread error message (checked on the host in
test_abi_host.py)."""
import threading

import pytest
import torch

from parity import require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _job(seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    L, Hq, Hkv, W, N, D, k = 1, 8, 2, 32, 3000 + 17 * seed, 128, 300
    U = L * Hkv
    return dict(q=torch.randn((L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16),
                k=torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16),
                scores=torch.empty((U, N), device=dev), kept=torch.empty((U, k), dtype=torch.int32, device=dev),
                k_total=k)


def _run(job, stream):
    ws = kv.score_window(job["q"], job["k"], job["scores"], stream=stream)
    kv.select(job["scores"], job["kept"], k_total=job["k_total"], n_sink=4, n_recent=16, pool="avg", pool_k=5,
              stream=stream)
    return ws


def test_threads_on_separate_streams_match_sequential_runs():
    dev = require_gpu()
    jobs = [_job(s, dev) for s in range(6)]
    for j in jobs:
        _run(j, None)
    torch.cuda.synchronize()
    want = [(j["scores"].clone(), j["kept"].clone()) for j in jobs]
    for j in jobs:
        j["scores"].fill_(float("nan"))
        j["kept"].fill_(-7)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in jobs]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    _run(jobs[i], streams[i])
            streams[i].synchronize()
        except Exception as e:                        # reported on the main thread
            errors.append(e)

    print("streams: 6 threads", flush=True)
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, (s, kept) in zip(jobs, want):
        assert torch.equal(j["scores"].view(torch.int32), s.view(torch.int32))
        assert torch.equal(j["kept"], kept)

