"""KVSEL_DEBUG=1: every call synchronises; NaN or Inf in a score array (the
scores a selection reads, the scores a scoring call writes) is reported as
E_ARG instead of being ranked silently; and the index lists that in-place
updates rely on (ascending block lists and distinct pages of the incremental
view, blocks shared between requests in a compaction, a request listed twice
for the ActKV scorer or keep score) are checked on the host before anything
runs.  The mode is read once per process, so the checks run in a child
process with the variable set."""
import os
import subprocess
import sys

import pytest

from parity import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
import selection_score_amd as kv
from selection_score_amd import _abi

dev = torch.device("cuda:0")
g = torch.Generator(device=dev).manual_seed(9)

def expect_error(fn, what, text="NaN or Inf"):
    try:
        fn()
    except kv.KvselError as e:
        assert e.status == _abi.KVSEL_E_ARG and text in str(e), str(e)
        print("caught", what, flush=True)
        return
    raise AssertionError(what + ": no error")

U, N, k = 4, 3000, 100
sc = torch.rand((U, N), generator=g, device=dev)
kept = torch.empty((U, k), dtype=torch.int32, device=dev)
ws = kv.select(sc, kept, k_total=k, n_sink=4, n_recent=8)
torch.cuda.synchronize()
print("clean select ok", flush=True)
sc[2, 1234] = float("nan")
expect_error(lambda: kv.select(sc, kept, k_total=k, n_sink=4, n_recent=8, workspace=ws), "select nan")
sc[2, 1234] = float("-inf")
expect_error(lambda: kv.select(sc, kept, k_total=k, n_sink=4, n_recent=8, workspace=ws), "select inf")

L, Hq, Hkv, W, D = 1, 4, 2, 16, 64
q = torch.randn((L, Hq, W, D), generator=g, device=dev).to(torch.bfloat16)
kk = torch.randn((L, Hkv, N, D), generator=g, device=dev).to(torch.bfloat16)
out = torch.empty((L * Hkv, N), device=dev)
kv.score_window(q, kk, out)
torch.cuda.synchronize()
assert torch.isfinite(out).all()
print("clean window ok", flush=True)
kk[0, 1, 77, 5] = float("inf")
expect_error(lambda: kv.score_window(q, kk, out), "window inf key")

# incremental view: a page listed twice, then a block list out of order
U2, nb, k2, bt = 2, 64, 8, 32
rk = torch.randn((U2, nb * bt, 128), generator=g, device=dev).to(torch.bfloat16)
pk = torch.zeros((U2, 12, bt, 128), dtype=torch.bfloat16, device=dev)
pv = torch.zeros_like(pk)
pt = torch.empty((U2, k2), dtype=torch.int32, device=dev)
nm = torch.empty(U2, dtype=torch.int32, device=dev)
new = torch.arange(0, 2 * k2, 2, dtype=torch.int32, device=dev).repeat(U2, 1).contiguous()
prev = torch.arange(1, 2 * k2, 2, dtype=torch.int32, device=dev).repeat(U2, 1).contiguous()
page = torch.arange(k2, dtype=torch.int32, device=dev).repeat(U2, 1).contiguous()
inc = lambda i, p: kv.gather_incremental(rk, rk, i, prev, p, pk, pv, pt, nm, bt=bt, D=128, src_rows=nb * bt,
                                         src_unit_stride=nb * bt * 128)
inc(new, page)
torch.cuda.synchronize()
print("clean incremental ok", flush=True)
bad_page = page.clone(); bad_page[1, 5] = 2
expect_error(lambda: inc(new, bad_page), "incremental page twice", "prev_page")
bad_new = new.clone(); bad_new[0, 3] = bad_new[0, 2]
expect_error(lambda: inc(bad_new, page), "incremental idx order", "idx of unit 0")

# compaction: one physical block in two requests
R, Y, bs, P = 2, 4, 16, 10
kp = torch.zeros((1, P, bs, 2, 64), dtype=torch.bfloat16, device=dev)
vp = torch.zeros_like(kp)
keep = torch.ones((R, Y * bs), dtype=torch.uint8, device=dev)
bt_tab = torch.arange(R * Y, dtype=torch.int32, device=dev).view(R, Y).contiguous()
outs = (torch.empty((R, Y * bs), dtype=torch.int32, device=dev), torch.empty((R, Y), dtype=torch.int32, device=dev),
        torch.empty(R, dtype=torch.int32, device=dev))
kv.compact(keep, bt_tab, kp, vp, *outs, block_size=bs)
torch.cuda.synchronize()
print("clean compact ok", flush=True)
bt_tab[1, 2] = 1
expect_error(lambda: kv.compact(keep, bt_tab, kp, vp, *outs, block_size=bs), "compact shared block", "block_table")

# ActKV scorer and keep score: a request listed twice
Ld, Rd, Hq2, Hkv2, Dd, n_cap = 1, 3, 8, 2, 128, 64
qd = torch.randn((Ld, 2, Hq2, Dd), generator=g, device=dev).to(torch.bfloat16)
lse = torch.zeros((Ld, 2, Hq2), device=dev) + 5.0
pool = torch.randn((Ld, 16, 16, Hkv2, Dd), generator=g, device=dev).to(torch.bfloat16)
btd = torch.arange(Rd * 4, dtype=torch.int32, device=dev).view(Rd, 4).contiguous()
n_ctx = torch.full((Rd,), 64, dtype=torch.int32, device=dev)
n_seen = torch.zeros(Rd, dtype=torch.int32, device=dev)
state = torch.zeros((Ld, Rd, Hkv2, n_cap), device=dev)
ks = torch.zeros((Rd, n_cap), device=dev)
ok_req = torch.tensor([0, 2], dtype=torch.int32, device=dev)
twice = torch.tensor([2, 2], dtype=torch.int32, device=dev)
kv.decode_score(qd, lse, pool, btd, n_ctx, n_seen, state, req=ok_req)
kv.keep_score(state, ks, n_ctx, lam=0.5, req=ok_req)
torch.cuda.synchronize()
print("clean actkv ok", flush=True)
expect_error(lambda: kv.decode_score(qd, lse, pool, btd, n_ctx, n_seen, state, req=twice), "decode req twice", "req")
expect_error(lambda: kv.keep_score(state, ks, n_ctx, lam=0.5, req=twice), "keep req twice", "req")
print("child done", flush=True)
"""


def test_debug_mode_reports_non_finite_scores():
    require_gpu()
    env = dict(os.environ, KVSEL_DEBUG="1", PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    print("debug mode: child process", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=100)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    for line in ("clean select ok", "caught select nan", "caught select inf", "clean window ok",
                 "caught window inf key", "clean incremental ok", "caught incremental page twice",
                 "caught incremental idx order", "clean compact ok", "caught compact shared block",
                 "clean actkv ok", "caught decode req twice", "caught keep req twice", "child done"):
        assert line in r.stdout
