// Session-memory attention scores over a paged KV pool.
//
// IntentKV §4 (rule score): each (layer, query head) of the session memory
// M attends over the history H with a softmax of M.K/sqrt(D); the rule score
// of a position sums those weights over all layers and heads.  The KV pool
// is paged (ActKV §2: physical page of logical page p = page_table[p]).
//
// Kernels:
//  1. logits: one workgroup per (layer, group of logical pages).  Each thread
//     keeps one query head's memory row in registers and dots it with K rows
//     of a page staged in LDS (double buffered, padded rows); logits go to a
//     float32 scratch [L][Hq][N] and each workgroup leaves a partial
//     (max, sum of exp) per head over the history positions it saw.  K is
//     read from HBM exactly once.
//  2. combine the partials into LSE[l][h].
//  3. per (layer, 256 positions): sum over the layer's heads of
//     exp(logit - LSE) over H -> per-layer partial rule (or the per-unit
//     output directly).
//  4. global: rule[j] = sum over layers in ascending order (deterministic).
#include "common.h"

#include <math.h>

namespace kvsel {

namespace {
constexpr int kPagesPerGroup = 16;
constexpr int kMaxHq = 64;

__device__ __forceinline__ bool in_history(const MemoryParams& p, int64_t j) {
  if (j < p.n_sink || j >= p.N - p.n_recent) return false;
  return p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[j]) != p.dead_slot;
}

struct WsLayout {
  size_t logits, part, lse, layer;   // byte offsets
  size_t total;
};

WsLayout ws_layout(const MemoryParams& p) {
  const int64_t n_lpages = ceil_div(p.N, p.page_size);
  const int64_t n_groups = ceil_div(n_lpages, kPagesPerGroup);
  WsLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.logits = take(static_cast<size_t>(p.L) * p.Hq * p.N * 4);
  w.part = take(static_cast<size_t>(p.L) * p.Hq * n_groups * 8);
  w.lse = take(static_cast<size_t>(p.L) * p.Hq * 4);
  w.layer = take(static_cast<size_t>(p.L) * p.N * 4);
  w.total = off;
  return w;
}
}  // namespace

size_t memory_workspace_bytes(const MemoryParams& p) { return ws_layout(p).total; }

template <int DT, int D>
__global__ __launch_bounds__(256) void memory_logits_kernel(MemoryParams p, const float* __restrict__ M,
                                                            const void* __restrict__ pool,
                                                            float* __restrict__ logits,
                                                            float2* __restrict__ part) {
  extern __shared__ __align__(16) uint8_t kbuf[];     // 2 x [page_size*Hkv][D*2 + 16]
  __shared__ float2 red[256];
  const int l = blockIdx.y, grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int G = p.Hq / p.Hkv;
  const int h = tid % p.Hq;
  const int g = h / G;
  const int slots = 256 / p.Hq;                       // token slots per pass
  const int row_bytes = D * 2 + 16;
  const int page_rows = p.page_size * p.Hkv;
  const int page_lds = page_rows * row_bytes;
  const int chunks_per_row = D * 2 / 16;
  const int64_t n_lpages = ceil_div(p.N, p.page_size);
  const int64_t lp_begin = static_cast<int64_t>(grp) * kPagesPerGroup;
  const int64_t lp_end = min(n_lpages, lp_begin + kPagesPerGroup);
  const int64_t layer_elems = p.pool_pages * p.page_size * p.Hkv * D;
  const uint8_t* lpool = static_cast<const uint8_t*>(pool) + static_cast<int64_t>(l) * layer_elems * 2;

  float mr[D];
  for (int d = 0; d < D; ++d) mr[d] = M[(static_cast<int64_t>(l) * p.Hq + h) * D + d];
  float m = -INFINITY, s = 0.f;

  auto load_page = [&](int64_t lp, uint8_t* dst) {
    const int64_t pp = p.page_table[lp];
    const bool ok = pp >= 0 && pp < p.pool_pages;
    const uint8_t* src = lpool + (ok ? pp : 0) * static_cast<int64_t>(page_rows) * D * 2;
    for (int c = tid; c < page_rows * chunks_per_row; c += 256) {
      const int row = c / chunks_per_row, piece = c % chunks_per_row;
      uint4 v = ok ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(row) * D * 2 + piece * 16)
                   : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(dst + row * row_bytes + piece * 16) = v;
    }
  };

  if (lp_begin < lp_end) load_page(lp_begin, kbuf);
  __syncthreads();
  for (int64_t lp = lp_begin; lp < lp_end; ++lp) {
    const int b = static_cast<int>(lp - lp_begin) & 1;
    if (lp + 1 < lp_end) load_page(lp + 1, kbuf + (b ^ 1) * page_lds);
    const uint8_t* buf = kbuf + b * page_lds;
    for (int o = tid / p.Hq; o < p.page_size; o += slots) {
      const int64_t j = lp * p.page_size + o;
      if (j >= p.N) break;
      const uint8_t* kr = buf + (o * p.Hkv + g) * row_bytes;
      float acc = 0.f;
      for (int d0 = 0; d0 < D; d0 += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(kr + d0 * 2);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        for (int i = 0; i < 4; ++i) {
          float lo, hi;
          if constexpr (DT == KVSEL_BF16) {
            lo = __uint_as_float(w4[i] << 16);
            hi = __uint_as_float(w4[i] & 0xFFFF0000u);
          } else {
            lo = f16_to_f32(static_cast<uint16_t>(w4[i] & 0xFFFFu));
            hi = f16_to_f32(static_cast<uint16_t>(w4[i] >> 16));
          }
          acc = fmaf(mr[d0 + 2 * i], lo, acc);
          acc = fmaf(mr[d0 + 2 * i + 1], hi, acc);
        }
      }
      const float x = acc * p.scale;
      logits[(static_cast<int64_t>(l) * p.Hq + h) * p.N + j] = x;
      if (in_history(p, j)) {
        if (x > m) {
          s = s * expf(m - x) + 1.f;
          m = x;
        } else {
          s += expf(x - m);
        }
      }
    }
    __syncthreads();
  }
  // combine the token slots that share head h
  red[tid] = make_float2(m, s);
  __syncthreads();
  if (tid < p.Hq) {
    float mm = -INFINITY, ss = 0.f;
    for (int k = 0; k < slots; ++k) {
      const float2 v = red[k * p.Hq + tid];
      if (v.x == -INFINITY) continue;
      const float mn = fmaxf(mm, v.x);
      ss = ((mm == -INFINITY) ? 0.f : ss * expf(mm - mn)) + v.y * expf(v.x - mn);
      mm = mn;
    }
    part[(static_cast<int64_t>(l) * p.Hq + tid) * gridDim.x + grp] = make_float2(mm, ss);
  }
}

__global__ void memory_lse_kernel(MemoryParams p, int n_groups, const float2* __restrict__ part,
                                  float* __restrict__ lse) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= p.L * p.Hq) return;
  float m = -INFINITY, s = 0.f;
  for (int gi = 0; gi < n_groups; ++gi) {
    const float2 v = part[static_cast<int64_t>(i) * n_groups + gi];
    if (v.x == -INFINITY) continue;
    const float mn = fmaxf(m, v.x);
    s = ((m == -INFINITY) ? 0.f : s * expf(m - mn)) + v.y * expf(v.x - mn);
    m = mn;
  }
  lse[i] = (m == -INFINITY) ? INFINITY : m + logf(s);   // empty history: every weight is 0
}

// per (256 positions, layer): sum over the layer's heads (global) or over each
// KV group's heads (per unit)
__global__ __launch_bounds__(256) void memory_rule_kernel(MemoryParams p, const float* __restrict__ logits,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ dst) {
  const int l = blockIdx.y;
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= p.N) return;
  const bool hist = in_history(p, j);
  const int G = p.Hq / p.Hkv;
  float acc = 0.f;
  for (int h = 0; h < p.Hq; ++h) {
    const float x = logits[(static_cast<int64_t>(l) * p.Hq + h) * p.N + j];
    acc += hist ? expf(x - lse[l * p.Hq + h]) : 0.f;
    if (p.reduce == KVSEL_REDUCE_PER_UNIT && (h % G) == G - 1) {
      dst[(static_cast<int64_t>(l) * p.Hkv + h / G) * p.N + j] = acc;
      acc = 0.f;
    }
  }
  if (p.reduce == KVSEL_REDUCE_GLOBAL) dst[static_cast<int64_t>(l) * p.N + j] = acc;
}

__global__ void memory_layer_sum_kernel(int L, int64_t N, const float* __restrict__ layer,
                                        float* __restrict__ out) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= N) return;
  float acc = 0.f;
  for (int l = 0; l < L; ++l) acc += layer[static_cast<int64_t>(l) * N + j];
  out[j] = acc;
}

template <int DT, int D>
static hipError_t launch_logits_t(const MemoryParams& p, int n_groups, const float* M,
                                  const void* pool, float* logits, float2* part, hipStream_t st) {
  const size_t sh = 2 * static_cast<size_t>(p.page_size) * p.Hkv * (D * 2 + 16);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&memory_logits_kernel<DT, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sh));
  if (e != hipSuccess) return e;
  dim3 grid(n_groups, p.L);
  memory_logits_kernel<DT, D><<<grid, 256, sh, st>>>(p, M, pool, logits, part);
  return hipGetLastError();
}

hipError_t launch_memory_scores(const MemoryParams& p, int dt, const float* M, const void* pool,
                                void* ws, float* out, hipStream_t st) {
  if (p.N == 0 || p.L == 0) return hipSuccess;
  const WsLayout w = ws_layout(p);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(base + w.logits);
  float2* part = reinterpret_cast<float2*>(base + w.part);
  float* lse = reinterpret_cast<float*>(base + w.lse);
  float* layer = reinterpret_cast<float*>(base + w.layer);
  const int n_groups = static_cast<int>(ceil_div(ceil_div(p.N, p.page_size), kPagesPerGroup));
  hipError_t e;
  if (dt == KVSEL_BF16) {
    e = (p.D == 64) ? launch_logits_t<KVSEL_BF16, 64>(p, n_groups, M, pool, logits, part, st)
                    : launch_logits_t<KVSEL_BF16, 128>(p, n_groups, M, pool, logits, part, st);
  } else {
    e = (p.D == 64) ? launch_logits_t<KVSEL_F16, 64>(p, n_groups, M, pool, logits, part, st)
                    : launch_logits_t<KVSEL_F16, 128>(p, n_groups, M, pool, logits, part, st);
  }
  if (e != hipSuccess) return e;
  memory_lse_kernel<<<static_cast<int>(ceil_div(p.L * p.Hq, 256)), 256, 0, st>>>(p, n_groups, part, lse);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(ceil_div(p.N, 256)), p.L);
  float* dst = (p.reduce == KVSEL_REDUCE_GLOBAL) ? layer : out;
  memory_rule_kernel<<<grid, 256, 0, st>>>(p, logits, lse, dst);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.reduce == KVSEL_REDUCE_GLOBAL) {
    memory_layer_sum_kernel<<<static_cast<int>(ceil_div(p.N, 256)), 256, 0, st>>>(p.L, p.N, layer, out);
    e = hipGetLastError();
  }
  return e;
}

static_assert(kMaxHq <= 256, "query heads per layer");

}  // namespace kvsel
