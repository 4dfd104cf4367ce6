"""KVSEL_DEBUG=1: every call synchronises, and NaN or Inf in a score array
(the scores a selection reads, the scores a scoring call writes) is reported
as E_ARG instead of being ranked silently.  The mode is read once per
process, so the checks run in a child process with the variable set."""
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

def expect_error(fn, what):
    try:
        fn()
    except kv.KvselError as e:
        assert e.status == _abi.KVSEL_E_ARG and "NaN or Inf" in str(e), str(e)
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
                 "caught window inf key", "child done"):
        assert line in r.stdout
