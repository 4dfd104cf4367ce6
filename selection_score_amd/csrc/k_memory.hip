// Session-memory attention scores over a paged KV pool.
//
// IntentKV §4 (rule score): each (layer, query head) of the session memory
// M attends over the history H with a softmax of M.K/sqrt(D); the rule score
// of a position sums those weights over all layers and heads.  The KV pool
// is paged (ActKV §2: physical page of logical page p = page_table[p]).
//
// Kernels:
//  1. logits: one workgroup per (layer, group of logical pages); logits go to
//     a float32 scratch [L][Hq][N] and each workgroup leaves a partial
//     (max, sum of exp) per head over the history positions it saw.  K is
//     read from HBM exactly once.  bf16 pools with D = 128, 16-token pages
//     and GQA groups of 4, 8 or 16 use the matrix cores
//     (memory_logits_mfma_kernel); other shapes dot on the vector ALUs with
//     pages staged in LDS (memory_logits_kernel).
//  2. combine the partials into LSE[l][h], one wavefront per (layer, head).
//  3. per (layer, 256 positions): sum over the layer's heads of
//     exp(logit - LSE) over H -> per-layer partial rule (or the per-unit
//     output directly).
//  4. global: rule[j] = sum over layers in ascending order (deterministic).
// Kernels 1-3 run once per group of layers, reusing one bounded logit
// scratch.
#include "common.h"

#include <math.h>

namespace kvsel {

namespace {
constexpr int kPagesPerGroup = 16;
// Logits -> LSE -> rule run in passes over groups of layers that reuse one
// logit scratch: as many layers per pass as the scratch the caller gave
// holds.  The workspace query asks for up to kScratchBytes (32 heads x 65536
// positions is 8 MiB per layer, so 36 layers take one pass).  Passes of a
// few layers, so that the scratch would stay in the Infinity Cache, were
// measured slower: the shorter launches lose more to their tails than the
// cache saves.
constexpr int64_t kScratchBytes = int64_t(512) << 20;

int64_t layer_scratch_bytes(const MemoryParams& p) { return (static_cast<int64_t>(p.Hq) * p.N * 4 + 255) / 256 * 256; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxHq = 64;

__device__ __forceinline__ bool in_history(const MemoryParams& p, int64_t j) {
  if (j < p.n_sink || j >= p.N - p.n_recent) return false;
  return p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[j]) != p.dead_slot;
}

struct WsLayout {
  size_t part, lse, layer;   // byte offsets of the fixed part
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
  w.part = take(static_cast<size_t>(p.L) * p.Hq * n_groups * 8);
  w.lse = take(static_cast<size_t>(p.L) * p.Hq * 4);
  w.layer = take(static_cast<size_t>(p.L) * p.N * 4);
  w.total = off;
  return w;
}
}  // namespace

size_t memory_fixed_bytes(const MemoryParams& p) { return ws_layout(p).total; }

size_t memory_logit_bytes(const MemoryParams& p, bool minimum) {
  const int64_t per = layer_scratch_bytes(p);
  if (minimum) return static_cast<size_t>(per);
  const int64_t layers = max(static_cast<int64_t>(1), min(static_cast<int64_t>(p.L), kScratchBytes / per));
  return static_cast<size_t>(layers * per);
}


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

// The logits on the matrix cores (bf16 pool, D = 128, 16-token pages, up to
// 32 query heads, GQA group G >= 4): v_mfma_f32_16x16x32_bf16 with the 16
// tokens of a page (one KV head) as A rows and 16 query heads as B columns;
// the columns of the KV head's own group are kept.  The float32 memory rows
// enter as bf16 hi + lo parts (about 16 significant bits; the logits keep
// ~2^-18 of the sum of |terms|).  Lane quarter q covers d = 32*ks + 8q .. +7
// of k-step ks on both operands.  Each wavefront serves one block of 16
// query heads (NG = 16 / G KV heads) and a share of the pages, reading all
// NG rows of a page straight into its A operands before multiplying.  The
// workgroup's logits (its 256 positions x Hq heads) are staged in LDS and
// written at the end as one 1 KiB run per head: the MFMA layout would
// otherwise scatter them in 64-byte pieces.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NCB, int NG>
__global__ __launch_bounds__(256) void memory_logits_mfma_kernel(MemoryParams p, const float* __restrict__ M,
                                                                 const void* __restrict__ pool,
                                                                 float* __restrict__ logits,
                                                                 float2* __restrict__ part) {
  constexpr int D = 128, PS = 16;
  constexpr int kWavesPerCb = 4 / NCB;
  constexpr int kRow = kPagesPerGroup * PS + 4;      // staged floats per head (padded)
  __shared__ float2 red[4][64];
  __shared__ __align__(16) float stage[32 * kRow];
  const int l = blockIdx.y, grp = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int cb = wave / kWavesPerCb, wsub = wave % kWavesPerCb;
  const int h = 16 * cb + col;                       // this lane's query head
  const int gi_own = col / G;                        // its KV head within the block
  // B operands: head h, d = 32*ks + 8*qd + j, as bf16 hi + lo
  bf16x8 bh[4], bl[4];
  {
    const float* row = M + (static_cast<int64_t>(l) * p.Hq + (h < p.Hq ? h : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (h < p.Hq) ? row[32 * ks + 8 * qd + j] : 0.f;
        const __bf16 hi = static_cast<__bf16>(x);
        bh[ks][j] = hi;
        bl[ks][j] = static_cast<__bf16>(x - static_cast<float>(hi));
      }
  }
  float m = -INFINITY, s = 0.f;
  const int64_t n_lpages = ceil_div(p.N, PS);
  const int64_t lp_begin = static_cast<int64_t>(grp) * kPagesPerGroup;
  const int64_t lp_end = min(n_lpages, lp_begin + kPagesPerGroup);
  const int64_t page_bytes = static_cast<int64_t>(PS) * p.Hkv * D * 2;
  const uint8_t* lpool = static_cast<const uint8_t*>(pool) + static_cast<int64_t>(l) * p.pool_pages * page_bytes;
  // the page table entry of the next page is read one page ahead
  int64_t pp_next = (lp_begin + wsub < lp_end) ? p.page_table[lp_begin + wsub] : -1;
  for (int64_t lp = lp_begin + wsub; lp < lp_end; lp += kWavesPerCb) {
    const int64_t pp = pp_next;
    if (lp + kWavesPerCb < lp_end) pp_next = p.page_table[lp + kWavesPerCb];
    const bool ok = pp >= 0 && pp < p.pool_pages;
    const uint8_t* base = lpool + (ok ? pp : 0) * page_bytes + (static_cast<int64_t>(col) * p.Hkv) * D * 2 + 16 * qd;
    uint4 a[NG][4];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int g = cb * NG + gi;
      const bool okg = ok && g < p.Hkv;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a[gi][ks] = okg ? *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(g) * D * 2 + 64 * ks)
                        : make_uint4(0, 0, 0, 0);
    }
    const int64_t j0 = lp * PS + 4 * qd;
    // history membership of this lane's four tokens, loaded with the page
    bool hist[4];
    {
      int32_t sm[4] = {0, 0, 0, 0};
      if (p.slot_map != nullptr) {
        if (j0 + 3 < p.N && (reinterpret_cast<uintptr_t>(p.slot_map) & 15) == 0) {
          const int4 v = *reinterpret_cast<const int4*>(p.slot_map + j0);
          sm[0] = v.x; sm[1] = v.y; sm[2] = v.z; sm[3] = v.w;
        } else {
          for (int i = 0; i < 4; ++i) sm[i] = (j0 + i < p.N) ? p.slot_map[j0 + i] : 0;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t j = j0 + i;
        hist[i] = j < p.N && j >= p.n_sink && j < p.N - p.n_recent &&
                  (p.slot_map == nullptr || static_cast<int64_t>(sm[i]) != p.dead_slot);
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a[gi][ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[ks], acc, 0, 0, 0);
      }
      // lane: head h, tokens 4*qd .. +3 of the page, kept if h is in KV head gi's group
      if (gi == gi_own && h < p.Hq) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = acc[i] * p.scale;
        *reinterpret_cast<float4*>(&stage[h * kRow + (lp - lp_begin) * PS + 4 * qd]) =
            make_float4(x[0], x[1], x[2], x[3]);
        for (int i = 0; i < 4; ++i) {
          if (!hist[i]) continue;
          if (x[i] > m) {
            s = s * __builtin_amdgcn_exp2f((m - x[i]) * kLog2e) + 1.f;
            m = x[i];
          } else {
            s += __builtin_amdgcn_exp2f((x[i] - m) * kLog2e);
          }
        }
      }
    }
  }
  // combine the lane quarters and the wavefronts that share a head
  red[wave][lane] = make_float2(m, s);
  __syncthreads();
  // the staged logits: whole rows of the group's positions, 16 bytes per lane
  {
    const int64_t j_begin = lp_begin * PS;
    const int n_pos = static_cast<int>(min(p.N, lp_end * PS) - j_begin);
    const int per_row = kRow / 4;                     // 16-byte pieces per staged row (incl. pad)
    for (int c = threadIdx.x; c < p.Hq * per_row; c += 256) {
      const int hh = c / per_row, jj = 4 * (c % per_row);
      if (jj >= n_pos) continue;
      const float4 v = *reinterpret_cast<const float4*>(&stage[hh * kRow + jj]);
      float* dst = logits + (static_cast<int64_t>(l) * p.Hq + hh) * p.N + j_begin + jj;
      if (jj + 3 < n_pos && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        // non-temporal: the scratch (Hq * N floats per layer) is read back
        // once per pass, and measured faster streamed past the caches
        typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(nt_f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<nt_f32x4*>(dst));
      } else {
        const float vv[4] = {v.x, v.y, v.z, v.w};
        for (int i = 0; i < 4 && jj + i < n_pos; ++i) dst[i] = vv[i];
      }
    }
  }
  if (threadIdx.x < 16 * NCB) {
    const int cbh = threadIdx.x / 16, c = threadIdx.x % 16;
    const int hh = 16 * cbh + c;
    float mm = -INFINITY, ss = 0.f;
    for (int w = cbh * kWavesPerCb; w < (cbh + 1) * kWavesPerCb; ++w)
      for (int q = 0; q < 4; ++q) {
        const float2 v = red[w][16 * q + c];
        if (v.x == -INFINITY) continue;
        const float mn = fmaxf(mm, v.x);
        ss = ((mm == -INFINITY) ? 0.f : ss * __builtin_amdgcn_exp2f((mm - mn) * kLog2e)) +
             v.y * __builtin_amdgcn_exp2f((v.x - mn) * kLog2e);
        mm = mn;
      }
    if (hh < p.Hq) part[(static_cast<int64_t>(l) * p.Hq + hh) * gridDim.x + grp] = make_float2(mm, ss);
  }
}

// One wavefront per (layer, head): lanes merge strided partials, then a
// fixed-order butterfly merges the lanes (deterministic).
__global__ __launch_bounds__(256) void memory_lse_kernel(MemoryParams p, int n_groups,
                                                         const float2* __restrict__ part,
                                                         float* __restrict__ lse) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x & 63;
  if (i >= p.L * p.Hq) return;                         // whole wavefronts leave together
  float m = -INFINITY, s = 0.f;
  for (int gi = lane; gi < n_groups; gi += 64) {
    const float2 v = part[static_cast<int64_t>(i) * n_groups + gi];
    if (v.x == -INFINITY) continue;
    const float mn = fmaxf(m, v.x);
    s = ((m == -INFINITY) ? 0.f : s * expf(m - mn)) + v.y * expf(v.x - mn);
    m = mn;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const float mn = fmaxf(m, m2);
    if (mn != -INFINITY) {
      s = ((m == -INFINITY) ? 0.f : s * expf(m - mn)) + ((m2 == -INFINITY) ? 0.f : s2 * expf(m2 - mn));
      m = mn;
    }
  }
  if (lane == 0) lse[i] = (m == -INFINITY) ? INFINITY : m + logf(s);   // empty history: every weight is 0
}

// per (1024 positions, layer): sum over the layer's heads (global) or over
// each KV group's heads (per unit), in head order; each thread takes four
// consecutive positions with 16-byte loads
__global__ __launch_bounds__(256) void memory_rule_kernel(MemoryParams p, const float* __restrict__ logits,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ dst) {
  const int l = blockIdx.y;
  const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (j0 >= p.N) return;
  const bool vec = (p.N % 4) == 0 && ((reinterpret_cast<uintptr_t>(logits) |
                                       reinterpret_cast<uintptr_t>(dst)) & 15) == 0;   // aligned rows, j0 + 3 < N
  bool hist[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) hist[i] = j0 + i < p.N && in_history(p, j0 + i);
  const int G = p.Hq / p.Hkv;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto put = [&](float* row) {
    if (vec) {
      *reinterpret_cast<float4*>(row + j0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      for (int i = 0; i < 4; ++i)
        if (j0 + i < p.N) row[j0 + i] = acc[i];
    }
  };
#pragma unroll 8
  for (int h = 0; h < p.Hq; ++h) {
    const float* row = logits + (static_cast<int64_t>(l) * p.Hq + h) * p.N;
    float x[4];
    if (vec) {
      const float4 v = *reinterpret_cast<const float4*>(row + j0);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else {
      for (int i = 0; i < 4; ++i) x[i] = (j0 + i < p.N) ? row[j0 + i] : 0.f;
    }
    const float ls = lse[l * p.Hq + h];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += hist[i] ? __builtin_amdgcn_exp2f((x[i] - ls) * kLog2e) : 0.f;
    if (p.reduce == KVSEL_REDUCE_PER_UNIT && (h % G) == G - 1) {
      put(dst + (static_cast<int64_t>(l) * p.Hkv + h / G) * p.N);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = 0.f;
    }
  }
  if (p.reduce == KVSEL_REDUCE_GLOBAL) put(dst + static_cast<int64_t>(l) * p.N);
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
                                void* ws, float* logits, size_t logit_bytes, float* out, hipStream_t st) {
  if (p.N == 0 || p.L == 0) return hipSuccess;
  const WsLayout w = ws_layout(p);
  uint8_t* base = static_cast<uint8_t*>(ws);
  float2* part_all = reinterpret_cast<float2*>(base + w.part);
  float* lse_all = reinterpret_cast<float*>(base + w.lse);
  float* layer = reinterpret_cast<float*>(base + w.layer);
  const int n_groups = static_cast<int>(ceil_div(ceil_div(p.N, p.page_size), kPagesPerGroup));
  const int G = p.Hq / p.Hkv;
  const int64_t layer_pool_bytes = p.pool_pages * p.page_size * p.Hkv * p.D * 2;
  hipError_t e;
  const int lpp = static_cast<int>(min(static_cast<int64_t>(p.L),
                                      static_cast<int64_t>(logit_bytes) / layer_scratch_bytes(p)));
  if (lpp < 1) return hipErrorInvalidValue;           // the caller checks the scratch holds one layer
  for (int l0 = 0; l0 < p.L; l0 += lpp) {
    // layers [l0, l0 + Lg) as a call of Lg layers on offset pointers
    MemoryParams q = p;
    q.L = min(lpp, p.L - l0);
    const float* Mq = M + static_cast<int64_t>(l0) * p.Hq * p.D;
    const void* poolq = static_cast<const uint8_t*>(pool) + l0 * layer_pool_bytes;
    float2* part = part_all + static_cast<int64_t>(l0) * p.Hq * n_groups;
    float* lse = lse_all + static_cast<int64_t>(l0) * p.Hq;
    if (dt == KVSEL_BF16 && p.D == 128 && p.page_size == 16 && p.Hq <= 32 && (G == 4 || G == 8 || G == 16)) {
      dim3 grid(n_groups, q.L);
#define KVSEL_MLM(NCB)                                                                     \
  do {                                                                                     \
    if (G == 4) memory_logits_mfma_kernel<NCB, 4><<<grid, 256, 0, st>>>(q, Mq, poolq, logits, part); \
    else if (G == 8) memory_logits_mfma_kernel<NCB, 2><<<grid, 256, 0, st>>>(q, Mq, poolq, logits, part); \
    else memory_logits_mfma_kernel<NCB, 1><<<grid, 256, 0, st>>>(q, Mq, poolq, logits, part); \
  } while (0)
      if (p.Hq <= 16) KVSEL_MLM(1);
      else KVSEL_MLM(2);
#undef KVSEL_MLM
      e = hipGetLastError();
    } else if (dt == KVSEL_BF16) {
      e = (p.D == 64) ? launch_logits_t<KVSEL_BF16, 64>(q, n_groups, Mq, poolq, logits, part, st)
                      : launch_logits_t<KVSEL_BF16, 128>(q, n_groups, Mq, poolq, logits, part, st);
    } else {
      e = (p.D == 64) ? launch_logits_t<KVSEL_F16, 64>(q, n_groups, Mq, poolq, logits, part, st)
                      : launch_logits_t<KVSEL_F16, 128>(q, n_groups, Mq, poolq, logits, part, st);
    }
    if (e != hipSuccess) return e;
    memory_lse_kernel<<<static_cast<int>(ceil_div(q.L * q.Hq, 4)), 256, 0, st>>>(q, n_groups, part, lse);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 grid(static_cast<unsigned>(ceil_div(p.N, 1024)), q.L);
    float* dst = (p.reduce == KVSEL_REDUCE_GLOBAL) ? layer + static_cast<int64_t>(l0) * p.N
                                                   : out + static_cast<int64_t>(l0) * p.Hkv * p.N;
    memory_rule_kernel<<<grid, 256, 0, st>>>(q, logits, lse, dst);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.reduce == KVSEL_REDUCE_GLOBAL) {
    memory_layer_sum_kernel<<<static_cast<int>(ceil_div(p.N, 256)), 256, 0, st>>>(p.L, p.N, layer, out);
    e = hipGetLastError();
  }
  return e;
}

static_assert(kMaxHq <= 256, "query heads per layer");

}  // namespace kvsel
