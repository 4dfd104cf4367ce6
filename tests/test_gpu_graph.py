"""The library's calls can be captured in a HIP graph and replayed.

Every call enqueues kernels only (no memset, copy or allocation), on the
stream it is given, with workspaces supplied by the caller.  A captured
SnapKV-style step (LSE pass, score pass, pooled select, gather) and a
captured ActKV decode token plus keep score are replayed several times,
with eager work and synchronisations between the replays, and every
replay must equal the eager result bit for bit.
"""
import pytest
import torch

from parity import require_gpu

import selection_score_amd as kv

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype.is_floating_point:
        return t.view(torch.int32 if t.element_size() == 4 else torch.int16)
    return t


def _replay_and_compare(graph, outputs, want, noise, fills=None):
    fills = fills or [7] * len(outputs)
    for rep in range(3):
        for o, f in zip(outputs, fills):
            o.fill_(f)                                # what each replay overwrites is scrambled first
        noise.mul_(1.5).add_(1.0)                    # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(_bits(o), _bits(w)), "replay %d differs" % rep


def test_snapkv_step_in_a_graph():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(5)
    L, Hq, Hkv, W, N, D, k = 2, 8, 2, 64, 4096, 128, 512
    U = L * Hkv
    q = torch.randn((L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
    kk = torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16)
    vv = torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16)
    lse = torch.empty((L, Hq, W), device=dev)
    scores = torch.empty((U, N), device=dev)
    kept = torch.empty((U, k), dtype=torch.int32, device=dev)
    dk = torch.empty((U, k, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty_like(dk)
    noise = torch.ones(1 << 20, device=dev)

    ws = {}

    def step():
        ws["lse"] = kv.score_window(q, kk, None, lse_out=lse, workspace=ws.get("lse"))
        kv.score_window(q, kk, scores, lse_in=lse)
        ws["sel"] = kv.select(scores, kept, k_total=k, n_sink=4, n_recent=64, pool="max", pool_k=7,
                              workspace=ws.get("sel"))
        kv.gather_rerope(kk.view(U, N, D), vv.view(U, N, D), kept, dk, dv, bt=1, D=D, src_rows=N,
                         src_unit_stride=N * D)

    print("graph: snapkv step eager", flush=True)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (lse, scores, kept, dk, dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                        # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("graph: capture", flush=True)
    with torch.cuda.graph(graph):
        step()
    print("graph: replays", flush=True)
    _replay_and_compare(graph, [lse, scores, kept, dk, dv], want, noise)


def test_actkv_decode_and_keep_score_in_a_graph():
    dev = require_gpu()
    g = torch.Generator(device=dev).manual_seed(6)
    L, R, Hq, Hkv, D, bs, N = 2, 3, 32, 8, 128, 16, 640
    Y = N // bs
    P = R * Y + 2
    q = torch.randn((L, R, Hq, D), generator=g, device=dev).to(torch.bfloat16)
    pool = torch.randn((L, P, bs, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    bt = torch.randperm(P, generator=g, device=dev)[: R * Y].view(R, Y).to(torch.int32)
    lse = torch.randn((L, R, Hq), generator=g, device=dev) + 8.0
    n_ctx = torch.tensor([640, 300, 17], dtype=torch.int32, device=dev)
    n_seen = torch.zeros(R, dtype=torch.int32, device=dev)      # a region start: the state is overwritten
    state = torch.empty((L, R, Hkv, N), device=dev)
    ks = torch.zeros((R, N), device=dev)
    attn = torch.empty((R, N), device=dev)
    hit = torch.empty((R, N), dtype=torch.uint8, device=dev)
    ws_keep = torch.empty(R * N * 4, dtype=torch.uint8, device=dev)
    noise = torch.ones(1 << 20, device=dev)

    def step():
        kv.decode_score(q, lse, pool, bt, n_ctx, n_seen, state)
        # lambda = 0: the keep score is hit * score, whatever it held before
        kv.keep_score(state, ks, n_ctx, lam=0.0, top_p=0.9, attn_score=attn, hit=hit, workspace=ws_keep)

    print("graph: actkv eager", flush=True)
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (state, ks, attn, hit)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    # entries past a request's length keep their keep score, so that buffer is
    # reset to its eager starting value rather than scrambled
    _replay_and_compare(graph, [state, ks, attn, hit], want, noise, fills=[7, 0, 7, 7])
