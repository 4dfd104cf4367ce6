"""GPU parity of kvsel_build_index (the Mean-K index of KVMem's block
retrieval) against the oracle's mean_k_index: fp16 bit patterns must match
exactly."""
import numpy as np
import pytest
import torch

from oracle import numerics
from oracle import score as osc
from parity import require_gpu

import selection_score_amd as kv
from selection_score_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_bits(raw_units, bt):
    """raw_units: list of float64 [rows][D] arrays -> uint16 [U][NB][D]."""
    return np.stack([numerics.f16_bits(osc.mean_k_index(r, bt)) for r in raw_units])


@pytest.mark.parametrize("dtype,D,bt,NB,b_begin,b_count", [
    (torch.bfloat16, 128, 32, 40, 0, 40),      # the KVMem block shape
    (torch.bfloat16, 64, 32, 9, 3, 5),         # append: a middle range only
    (torch.float16, 128, 7, 13, 0, 13),        # rows per block not a multiple of a wave pass
    (torch.float32, 128, 32, 6, 1, 4),
    (torch.float32, 64, 1, 50, 0, 50),         # one row per block: the row itself, rounded
    (torch.bfloat16, 128, 256, 3, 0, 3),       # the largest block
])
def test_index_matches_oracle(dtype, D, bt, NB, b_begin, b_count):
    dev = require_gpu()
    rng = np.random.default_rng(D * 1000 + bt)
    U = 5
    rows = NB * bt + 3                          # a trailing partial block is never indexed
    raw = torch.from_numpy(rng.standard_normal((U, rows, D)) * rng.choice([1e-3, 1.0, 300.0], size=(U, rows, 1)))
    raw = raw.to(dtype).to(dev)
    mu = torch.full((U, NB, D), 7.0, dtype=torch.float16, device=dev)
    kv.build_index(raw, mu, bt=bt, D=D, src_rows=rows, src_unit_stride=rows * D, b_begin=b_begin, b_count=b_count)
    torch.cuda.synchronize()
    got = _bits16(mu)
    want = _oracle_bits([raw[u].double().cpu().numpy() for u in range(U)], bt)
    lo, hi = b_begin, b_begin + b_count
    np.testing.assert_array_equal(got[:, lo:hi], want[:, lo:hi])
    untouched = np.concatenate([got[:, :lo], got[:, hi:]], axis=1)
    assert np.all(untouched == numerics.f16_bits(7.0))


def test_index_rounding_edges_and_signed_zero():
    # float32 rows: means exactly halfway between halves go to the even one,
    # beyond 65520 to inf; a sum that starts from 0 makes a block of negative
    # zeros +0
    dev = require_gpu()
    u = 2.0 ** -10
    D = 64
    col = np.array([1.0, 1.0 + u,            # -> 1.0
                    1.0 + u, 1.0 + 2 * u,    # -> 1 + 2u
                    70000.0, 70000.0,        # -> inf
                    -0.0, -0.0,              # -> +0
                    -1.0, 1.0,               # -> +0
                    2.0 ** -25, 2.0 ** -25])  # below half the smallest subnormal -> 0
    raw = np.repeat(col[:, None], D, axis=1)
    t = torch.from_numpy(raw.astype(np.float32))[None].to(dev)
    mu = torch.empty((1, 6, D), dtype=torch.float16, device=dev)
    kv.build_index(t, mu, bt=2, D=D, src_rows=12, src_unit_stride=12 * D)
    torch.cuda.synchronize()
    got = _bits16(mu)[0, :, 0]
    np.testing.assert_array_equal(got, _oracle_bits([raw], 2)[0, :, 0])
    np.testing.assert_array_equal(got, [0x3C00, 0x3C02, 0x7C00, 0x0000, 0x0000, 0x0000])


def test_index_aliased_units_through_offsets():
    # units read shared layer buffers through per-unit element offsets, as the
    # raw store of the 1M-token workspace does
    dev = require_gpu()
    rng = np.random.default_rng(5)
    n_buf, Hkv, NB, bt, D = 2, 2, 6, 32, 128
    store = torch.from_numpy(rng.standard_normal((n_buf, Hkv, NB * bt, D))).to(torch.bfloat16).to(dev)
    L = 4
    offs = torch.tensor([((l % n_buf) * Hkv + h) * NB * bt * D for l in range(L) for h in range(Hkv)],
                        dtype=torch.int64, device=dev)
    mu = torch.empty((L * Hkv, NB, D), dtype=torch.float16, device=dev)
    kv.build_index(store, mu, bt=bt, D=D, src_rows=NB * bt, src_offsets=offs)
    torch.cuda.synchronize()
    got = _bits16(mu)
    s = store.double().cpu().numpy()
    want = _oracle_bits([s[l % n_buf, h] for l in range(L) for h in range(Hkv)], bt)
    np.testing.assert_array_equal(got, want)


def test_index_empty_calls():
    dev = require_gpu()
    mu = torch.full((2, 4, 64), 3.0, dtype=torch.float16, device=dev)
    raw = torch.zeros((2, 128, 64), dtype=torch.bfloat16, device=dev)
    kv.build_index(raw, mu, bt=32, D=64, src_rows=128, src_unit_stride=128 * 64, b_begin=2, b_count=0)
    torch.cuda.synchronize()
    assert torch.all(mu == 3.0)
    with pytest.raises(kv.KvselError):
        kv.build_index(raw, mu, bt=32, D=64, src_rows=100, src_unit_stride=128 * 64)   # past src_rows


def test_index_1m_workspace_full_size_sampled():
    """The whole 1M-token index (64 layers x 8 KV heads x 32768 blocks of 32
    raw bf16 rows) in the launch configuration the benchmark times; sampled
    blocks of sampled units against the oracle, the rest by a property."""
    dev = require_gpu()
    cfg = wl.CONFIGS["kvmem1m"]
    raw_k, _, offs = wl.kvmem_raw_store(cfg, dev)
    U, NB, bt, D = cfg.U, cfg.N, cfg.bt, cfg.D
    mu = torch.empty((U, NB, D), dtype=torch.float16, device=dev)
    kv.build_index(raw_k, mu, bt=bt, D=D, src_rows=NB * bt, src_offsets=offs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    offs_h = offs.cpu().numpy()
    flat = raw_k.view(-1)
    for u in [0, 77, U - 1]:
        blocks = np.sort(rng.choice(NB, 256, replace=False))
        rows = (blocks[:, None] * bt + np.arange(bt)[None]).reshape(-1)
        base = int(offs_h[u])
        sel = flat[base: base + NB * bt * D].view(NB * bt, D)[torch.from_numpy(rows).to(dev)]
        want = numerics.f16_bits(osc.mean_k_index(sel.double().cpu().numpy(), bt))
        got = _bits16(mu[u][torch.from_numpy(blocks).to(dev)])
        np.testing.assert_array_equal(got, want)
    # layers that alias one raw buffer hold identical indexes
    assert torch.equal(mu[0].view(torch.int16), mu[cfg.raw_layers * cfg.Hkv].view(torch.int16))
    assert torch.isfinite(mu.float()).all()
