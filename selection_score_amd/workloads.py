"""Seeded synthetic inputs with the shapes of the five selection workloads.

Shared by the parity tests (which hand the same tensors to the HIP path and
to the CPU oracle) and by ``bench.py``.  Nothing here computes any step of
the selection method: these functions only draw random tensors with the
stated structure and round them to the storage dtype.

Workloads (shapes of the settings the three pages describe):
  tiny        1 layer, 2 KV / 8 query heads, D 64, fp32, N 2048, window 16,
              16 planted keys scaled x8, avg-pool 7, budget 512 (4 sink, 64 recent)
  snapkv      36 layers, 8 KV / 32 query heads, D 128, bf16, N 32768, window 64,
              rank-8 per-unit structure, max-pool 7, per-head budget 8192 (4 + 256)
  intentkv    36 layers, 8 KV / 32 query heads, D 128, bf16 paged pool (16-token
              pages, random physical order, sentinel page last), N 65536, 8 turns
              of 64 queries, budget 8192 (4 sink + 64 recent), decay 0.9
  kvmem1m     64 layers, 8 KV / 64 query heads, D 128, 32768 32-token blocks per
              unit, fp16 Mean-K index, 512-token bf16 query, top 2048 blocks
              (block 0 + last 4 forced), raw K/V in 8 aliased layer buffers, theta 1e6
  kvmem10m    same model, 312500 blocks per unit scored in 65536-block tiles,
              4 sessions, 4096-block views, 50% overlap with the previous view
  actkv       in-place tail compaction of paged KV: 64 requests of 6144 positions
              in 16-slot blocks compressed to 4096 kept entries (4 sink + 64
              recent + the rest drawn denser toward the tail), 36 layers of
              8 KV heads, D 128, bf16 pools; the same shape for the action
              scorer's running means (5 action tokens already folded in), the
              LRFU keep score (lambda 0.5, top-p 0.9) and one decode token of
              the recovery scorer over all 64 requests (32 query heads)
"""
import dataclasses
import math

import torch


@dataclasses.dataclass
class Config:
    name: str
    seed: int
    L: int
    Hkv: int
    Hq: int
    D: int
    N: int                 # tokens (token workloads) or blocks per unit (block workloads)
    k: int                 # budget per selection unit
    n_sink: int
    n_recent: int
    dtype: torch.dtype = torch.bfloat16
    W: int = 0             # window rows / query tokens per head
    pool: str = "none"
    pool_k: int = 1
    page_size: int = 16
    turns: int = 0
    decay: float = 0.9
    bt: int = 32
    theta: float = 1e6
    raw_layers: int = 8
    S: int = 1
    tile: int = 0
    planted: int = 0
    plant_scale: float = 8.0

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def U(self):
        return self.L * self.Hkv


CONFIGS = {
    "tiny": Config("tiny", 1001, L=1, Hkv=2, Hq=8, D=64, N=2048, k=512, n_sink=4, n_recent=64,
                   dtype=torch.float32, W=16, pool="avg", pool_k=7, planted=16),
    "snapkv": Config("snapkv", 1002, L=36, Hkv=8, Hq=32, D=128, N=32768, k=8192, n_sink=4,
                     n_recent=256, W=64, pool="max", pool_k=7),
    "intentkv": Config("intentkv", 1003, L=36, Hkv=8, Hq=32, D=128, N=65536, k=8192, n_sink=4,
                       n_recent=64, W=64, turns=8, page_size=16),
    "kvmem1m": Config("kvmem1m", 1004, L=64, Hkv=8, Hq=64, D=128, N=32768, k=2048, n_sink=1,
                      n_recent=4, dtype=torch.bfloat16, W=512, bt=32, theta=1e6, raw_layers=8),
    "kvmem10m": Config("kvmem10m", 1005, L=64, Hkv=8, Hq=64, D=128, N=312500, k=4096, n_sink=1,
                       n_recent=4, dtype=torch.bfloat16, W=512, bt=32, theta=1e6, raw_layers=1,
                       S=4, tile=65536),
    "actkv": Config("actkv", 1006, L=36, Hkv=8, Hq=32, D=128, N=6144, k=4096, n_sink=4, n_recent=64,
                    page_size=16, S=64, turns=5, decay=0.5),
}


def _gen(cfg, device, salt=0):
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1000 + salt)
    return g


def _randn(shape, g, device, std=1.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


# ------------------------------------------------------------------ token windows

def tiny_inputs(cfg, device):
    """K, V, Q ~ N(0,1) (float32); `planted` positions drawn without
    replacement from [4, N-64) have their keys scaled by `plant_scale`."""
    g = _gen(cfg, device)
    k = _randn((cfg.L, cfg.Hkv, cfg.N, cfg.D), g, device)
    v = _randn((cfg.L, cfg.Hkv, cfg.N, cfg.D), g, device)
    q = _randn((cfg.L, cfg.Hq, cfg.W, cfg.D), g, device)
    lo, hi = 4, max(5, cfg.N - 64)
    perm = torch.randperm(hi - lo, generator=g, device=device)[: cfg.planted] + lo
    planted = torch.sort(perm).values
    k[:, :, planted] *= cfg.plant_scale
    return dict(q=q.to(cfg.dtype), k=k.to(cfg.dtype), v=v.to(cfg.dtype), planted=planted)


def _lowrank_keys(cfg, g, device, basis):
    """Per unit: K_j = e_j + c_j B_u with e ~ N(0, I), c_j ~ N(0, I_8)."""
    L, Hkv, N, D = cfg.L, cfg.Hkv, cfg.N, cfg.D
    out = torch.empty((L, Hkv, N, D), dtype=cfg.dtype, device=device)
    for l in range(L):
        e = _randn((Hkv, N, D), g, device)
        c = _randn((Hkv, N, basis.shape[2]), g, device)
        out[l] = (e + torch.bmm(c, basis[l])).to(cfg.dtype)
    return out


def snapkv_inputs(cfg, device, rank=8):
    """Keys with per-unit rank-`rank` structure (basis B_u ~ N(0, I/rank)),
    window queries built the same way from the basis of their KV group,
    V ~ N(0,1); all bf16."""
    g = _gen(cfg, device)
    basis = _randn((cfg.L, cfg.Hkv, rank, cfg.D), g, device, std=1.0 / math.sqrt(rank))
    k = _lowrank_keys(cfg, g, device, basis)
    v = torch.empty_like(k)
    for l in range(cfg.L):
        v[l] = _randn((cfg.Hkv, cfg.N, cfg.D), g, device).to(cfg.dtype)
    grp = torch.arange(cfg.Hq, device=device) // cfg.G
    eq = _randn((cfg.L, cfg.Hq, cfg.W, cfg.D), g, device)
    cq = _randn((cfg.L, cfg.Hq, cfg.W, rank), g, device)
    q = (eq + torch.matmul(cq, basis[:, grp])).to(cfg.dtype)
    return dict(q=q, k=k, v=v)


# ------------------------------------------------------------------ session memory, paged

def intentkv_inputs(cfg, device, rank=8):
    """Paged pool [L][P+1][page][Hkv][D] bf16 (pages in a seeded random
    physical order, page P reserved for the dead slot), K as in `snapkv`
    plus sqrt(D) * r_j * u_(l,g) with a per-token relevance r shared by every
    (l, g) and unit intent directions u in the span of the basis; V ~ N(0,1);
    `turns` turns of W query rows N(0, I) + 4 u_(l,g(h)) with a per-turn drift
    of the direction (0.3 N(0, I) before normalising)."""
    g = _gen(cfg, device)
    L, Hkv, N, D, ps = cfg.L, cfg.Hkv, cfg.N, cfg.D, cfg.page_size
    n_pages = (N + ps - 1) // ps
    P = n_pages + 1
    basis = _randn((L, Hkv, rank, D), g, device, std=1.0 / math.sqrt(rank))
    w = _randn((L, Hkv, 1, rank), g, device)
    u = torch.matmul(w, basis)[:, :, 0]
    u = u / u.norm(dim=-1, keepdim=True)
    r = _randn((N,), g, device)
    page_table = torch.randperm(n_pages, generator=g, device=device).to(torch.int32)
    j = torch.arange(N, device=device)
    slot_map = (page_table.long()[j // ps] * ps + j % ps).to(torch.int32)
    k_pool = torch.zeros((L, P, ps, Hkv, D), dtype=cfg.dtype, device=device)
    v_pool = torch.zeros_like(k_pool)
    pad = n_pages * ps - N
    for l in range(L):
        e = _randn((Hkv, N, D), g, device)
        c = _randn((Hkv, N, rank), g, device)
        kl = e + torch.bmm(c, basis[l]) + math.sqrt(D) * r[None, :, None] * u[l][:, None, :]
        vl = _randn((Hkv, N, D), g, device)
        if pad:
            kl = torch.cat([kl, torch.zeros((Hkv, pad, D), device=device)], dim=1)
            vl = torch.cat([vl, torch.zeros((Hkv, pad, D), device=device)], dim=1)
        # logical [Hkv][n_pages][ps][D] -> physical pages
        kl = kl.view(Hkv, n_pages, ps, D).permute(1, 2, 0, 3).to(cfg.dtype)
        vl = vl.view(Hkv, n_pages, ps, D).permute(1, 2, 0, 3).to(cfg.dtype)
        k_pool[l, page_table.long()] = kl
        v_pool[l, page_table.long()] = vl
    grp = torch.arange(cfg.Hq, device=device) // cfg.G
    turns = []
    for _ in range(cfg.turns):
        drift = u + 0.3 * _randn(u.shape, g, device)
        drift = drift / drift.norm(dim=-1, keepdim=True)
        qt = _randn((L, cfg.Hq, cfg.W, D), g, device) + 4.0 * drift[:, grp][:, :, None, :]
        turns.append(qt.to(cfg.dtype))
    dead_slot = n_pages * ps            # first slot of the reserved page
    return dict(k_pool=k_pool, v_pool=v_pool, page_table=page_table, slot_map=slot_map,
                turns=turns, dead_slot=dead_slot)


# ------------------------------------------------------------------ Mean-K blocks

def kvmem_index(cfg, device, n_dirs=1, planted=None):
    """fp16 Mean-K index [L][Hkv][N][D] = N(0, I/32) + sum over directions d of
    (r_d[u,b] / sqrt(D)) w_d[u], r ~ N(0,1), w unit vectors per unit.
    With `planted` = (count, level), each direction d also raises r_d on a
    seeded set of `count` non-forced blocks per unit by `level`; the sets are
    returned so a previous view can overlap a predictable part of the next."""
    g = _gen(cfg, device, salt=1)
    L, Hkv, NB, D = cfg.L, cfg.Hkv, cfg.N, cfg.D
    w = _randn((n_dirs, L, Hkv, D), g, device)
    w = w / w.norm(dim=-1, keepdim=True)
    mu = torch.empty((L, Hkv, NB, D), dtype=torch.float16, device=device)
    sets = None
    if planted is not None:
        count, level = planted
        sets = torch.empty((n_dirs, L, Hkv, count), dtype=torch.int32, device=device)
    chunk = 1 << 16
    for l in range(L):
        for h in range(Hkv):
            boost = torch.zeros((n_dirs, NB), device=device)
            if planted is not None:
                for d in range(n_dirs):
                    cand = torch.randperm(NB - cfg.n_sink - cfg.n_recent, generator=g,
                                          device=device)[:count] + cfg.n_sink
                    s = torch.sort(cand).values
                    sets[d, l, h] = s.to(torch.int32)
                    boost[d, s] = level
            for b0 in range(0, NB, chunk):
                b1 = min(NB, b0 + chunk)
                x = _randn((b1 - b0, D), g, device, std=1.0 / math.sqrt(32.0))
                r = _randn((n_dirs, b1 - b0), g, device) + boost[:, b0:b1]
                x += torch.einsum("nb,nd->bd", r, w[:, l, h]) / math.sqrt(D)
                mu[l, h, b0:b1] = x.to(torch.float16)
    return mu, w, sets


def kvmem_queries(cfg, device, w, session):
    """Pre-RoPE prefill queries [L][Hq][W][D] bf16 = N(0, I) + 2 w_session[u(h)]."""
    g = _gen(cfg, device, salt=10 + session)
    grp = torch.arange(cfg.Hq, device=device) // cfg.G
    q = _randn((cfg.L, cfg.Hq, cfg.W, cfg.D), g, device) + 2.0 * w[session][:, grp][:, :, None, :]
    return q.to(torch.bfloat16)


def kvmem_raw_store(cfg, device):
    """Raw (position-free) K and V, bf16, in `raw_layers` physical buffers of
    [Hkv][N][bt][D]; unit (l, g) reads buffer l mod raw_layers.  Returns the
    stores and the per-unit int64 element offsets."""
    g = _gen(cfg, device, salt=2)
    shape = (cfg.raw_layers, cfg.Hkv, cfg.N, cfg.bt, cfg.D)
    k = torch.empty(shape, dtype=torch.bfloat16, device=device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for i in range(cfg.raw_layers):
        for h in range(cfg.Hkv):
            k[i, h] = _randn(shape[2:], g, device).to(torch.bfloat16)
            v[i, h] = _randn(shape[2:], g, device).to(torch.bfloat16)
    unit_elems = cfg.N * cfg.bt * cfg.D
    l = torch.arange(cfg.L, device=device)[:, None]
    h = torch.arange(cfg.Hkv, device=device)[None, :]
    offsets = (((l % cfg.raw_layers) * cfg.Hkv + h) * unit_elems).reshape(-1).to(torch.int64)
    return k, v, offsets


# ------------------------------------------------------------------ tail compaction

def actkv_inputs(cfg, device, spare_blocks=64):
    """S requests of N positions in page_size-slot blocks.  Keep masks: the
    n_sink first and n_recent last positions, plus k - n_sink - n_recent more
    drawn without replacement with weights exp(1.5 j / N) (denser toward the
    tail).  Block tables: a seeded permutation of the pool's blocks.  Pools
    [L][S*Y + spare][page_size][Hkv][D] ~ N(0, 1) in cfg.dtype."""
    g = _gen(cfg, device)
    R, N, bs = cfg.S, cfg.N, cfg.page_size
    Y = (N + bs - 1) // bs
    P = R * Y + spare_blocks
    keep = torch.zeros((R, N), dtype=torch.uint8, device=device)
    keep[:, : cfg.n_sink] = 1
    keep[:, N - cfg.n_recent:] = 1
    mid = torch.arange(cfg.n_sink, N - cfg.n_recent, device=device)
    w = torch.exp(1.5 * mid.double() / N)
    extra = cfg.k - cfg.n_sink - cfg.n_recent
    for r in range(R):
        pick = torch.multinomial(w, extra, replacement=False, generator=g)
        keep[r, mid[pick]] = 1
    block_table = torch.randperm(P, generator=g, device=device)[: R * Y].view(R, Y).to(torch.int32)
    k_pool = torch.empty((cfg.L, P, bs, cfg.Hkv, cfg.D), dtype=cfg.dtype, device=device)
    v_pool = torch.empty_like(k_pool)
    for l in range(cfg.L):
        k_pool[l] = _randn(k_pool.shape[1:], g, device).to(cfg.dtype)
        v_pool[l] = _randn(v_pool.shape[1:], g, device).to(cfg.dtype)
    return dict(keep=keep, block_table=block_table, k_pool=k_pool, v_pool=v_pool)


def actkv_state(cfg, device, salt=7):
    """Running means of an action region, [L][S][Hkv][N] float32: per
    (layer, request, KV head) row a softmax over positions of the logits
    1.5 * j / N + z[r, j] + N(0, 0.75^2), with z ~ N(0, 1.5^2) shared by every
    layer and head of a request (the same entries matter across heads), so
    the rows are heavy-tailed, denser toward the tail and sum to 1, as the
    recovery scorer leaves them."""
    g = _gen(cfg, device, salt)
    R, N = cfg.S, cfg.N
    ramp = 1.5 * torch.arange(N, device=device, dtype=torch.float32) / N
    shared = ramp + _randn((R, 1, N), g, device, std=1.5)
    st = torch.empty((cfg.L, R, cfg.Hkv, N), dtype=torch.float32, device=device)
    for l in range(cfg.L):
        st[l] = torch.softmax(shared + _randn((R, cfg.Hkv, N), g, device, std=0.75), dim=-1)
    return st


def actkv_decode_inputs(cfg, device, spare_blocks=64):
    """One decode token of every request for the recovery scorer.

    Keys carry a per-(request, position) relevance rel ~ N(0, 4^2) along one
    unit direction u[l, g] per (layer, KV head): K = e + rel * u with
    e ~ N(0, I), in a pool of [L][S*Y + spare][page_size][Hkv][D] in blocks of
    a seeded permutation.  Queries (post-RoPE) are N(0, I) + 8 u[l, g(h)], so
    the logits spread with a standard deviation near 3 and attention is
    heavy-tailed.  The LSE is what a paged attention pass returns for these
    queries: the float32 log-sum-exp of the scaled logits over the first
    n_ctx = N positions, computed here with torch on the device (input
    synthesis; the scorer only consumes it).  n_seen = cfg.turns action
    tokens are already in the state (``actkv_state``)."""
    g = _gen(cfg, device, 11)
    R, N, bs, L, Hkv, D, Hq = cfg.S, cfg.N, cfg.page_size, cfg.L, cfg.Hkv, cfg.D, cfg.Hq
    G = Hq // Hkv
    Y = (N + bs - 1) // bs
    P = R * Y + spare_blocks
    block_table = torch.randperm(P, generator=g, device=device)[: R * Y].view(R, Y).to(torch.int32)
    rel = _randn((R, Y * bs), g, device, std=4.0)
    # relevance of every physical slot (0 for the spare blocks)
    rel_phys = torch.zeros((P, bs), dtype=torch.float32, device=device)
    rel_phys[block_table.long().view(-1)] = rel.view(R * Y, bs)
    u = _randn((L, Hkv, D), g, device)
    u = u / u.norm(dim=-1, keepdim=True)
    k_pool = torch.empty((L, P, bs, Hkv, D), dtype=cfg.dtype, device=device)
    q = torch.empty((L, R, Hq, D), dtype=cfg.dtype, device=device)
    lse = torch.empty((L, R, Hq), dtype=torch.float32, device=device)
    scale = 1.0 / math.sqrt(D)
    for l in range(L):
        k_pool[l] = (_randn((P, bs, Hkv, D), g, device) + rel_phys[:, :, None, None] * u[l][None, None]).to(cfg.dtype)
        q[l] = (_randn((R, Hq, D), g, device) + 8.0 * u[l].repeat_interleave(G, dim=0)[None]).to(cfg.dtype)
        keys = k_pool[l][block_table.long()].reshape(R, Y * bs, Hkv, D)[:, :N].float()     # [R][N][Hkv][D]
        keys = keys.permute(0, 2, 1, 3).contiguous()                                       # [R][Hkv][N][D]
        qg = q[l].float().view(R, Hkv, G, D).transpose(2, 3).contiguous()                  # [R][Hkv][D][G]
        logits = torch.matmul(keys, qg) * scale                                            # [R][Hkv][N][G]
        lse[l] = torch.logsumexp(logits, dim=2).reshape(R, Hq)
        del keys, logits
    n_ctx = torch.full((R,), N, dtype=torch.int32, device=device)
    n_seen = torch.full((R,), cfg.turns, dtype=torch.int32, device=device)
    return dict(block_table=block_table, k_pool=k_pool, q=q, lse=lse, n_ctx=n_ctx, n_seen=n_seen)
