// ActKV decode-streaming action scorer and LRFU keep score.
//
// decode_score_kernel -- ActKV §7.1, Algorithm 3.  For the current query
//   token of each request that is generating an action, every cached key of
//   every KV head gets p = max over the group's query heads of
//   exp(scale * q.k - LSE), with the LSE taken from the paged attention pass,
//   and p is folded into a running mean over the action tokens of the
//   region.  Keys are read straight from the paged pool through the block
//   table.  One wavefront serves one (layer, request, KV head, 64 positions)
//   tile: four 16-key sub-pages, each multiplied on the matrix cores with
//   v_mfma_f32_16x16x32_{bf16,f16}, the group's query heads as A rows and the
//   sub-page's 16 keys as B columns.  The result lane (row 4*quarter + i,
//   column c) then holds head 4*quarter + i of key c, so the maximum over
//   a group of up to four heads is taken inside a lane.  The maximum is
//   taken on the logits (exp is monotone) and one exp2 per key follows.
//   Cost: the pool's keys are read once (HBM-bound); the state row is read
//   and written once.
//
// action_reduce_kernel + top_p_update_kernel -- ActKV §5.2.  At a
//   compression step each entry's action score is the sum over layers and
//   KV heads of the running means (compensated float64 sum, rounded once to
//   float32); the top-p set is the shortest prefix of the entries by score
//   (lower index first on ties) whose cumulative score reaches top_p times
//   the total, and the keep score becomes lambda * KS + hit * score.  The
//   top-p boundary is found by a radix descent over the float bits with
//   weight (not count) histograms: the entries of one 8-bit bucket lie within
//   a factor of four of each other, so every bucket sum below 2^28 entries is
//   exact in float64 whatever the order of the atomic adds.
#include "common.h"

namespace kvsel {

typedef __bf16 dec_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 dec_f16x8 __attribute__((ext_vector_type(8)));
typedef float dec_f32x4 __attribute__((ext_vector_type(4)));

constexpr float kDecLog2e = 1.4426950408889634f;
constexpr int kDecSubPages = 4;   // 16-key sub-pages per wavefront tile

template <int DT>
__device__ __forceinline__ dec_f32x4 dec_mfma(const uint4& a, const uint4& b, dec_f32x4 c) {
  if constexpr (DT == KVSEL_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dec_bf16x8, a),
                                                   __builtin_bit_cast(dec_bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(dec_f16x8, a),
                                                  __builtin_bit_cast(dec_f16x8, b), c, 0, 0, 0);
  }
}

template <int DT, int D>
__global__ __launch_bounds__(512) void decode_score_kernel(DecodeParams p, const void* __restrict__ q,
                                                           const float* __restrict__ lse,
                                                           const void* __restrict__ k_pool,
                                                           float* __restrict__ state) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int a = blockIdx.y, l = blockIdx.z;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int r = (p.req != nullptr) ? p.req[a] : a;
  if (r < 0 || r >= p.R) return;
  const int64_t n_lim = min(p.n_cap, static_cast<int64_t>(p.Y) * p.block_size);
  const int64_t n = min(max(static_cast<int64_t>(p.n_ctx[r]), static_cast<int64_t>(0)), n_lim);
  const int t = max(p.n_seen[r], 0);
  const float inv = 1.0f / (static_cast<float>(t) + 1.0f);   // no int overflow at n_seen = INT_MAX
  const int64_t j = j0 + lane;
  const int64_t jc = min(j, p.n_cap - 1);
  const int64_t row_elems = static_cast<int64_t>(p.Hkv) * D;
  const uint16_t* pool = static_cast<const uint16_t*>(k_pool);
  const int32_t* btab = p.block_table + static_cast<int64_t>(r) * p.Y;
  const int waves = blockDim.x >> 6;

  for (int g = wave; g < p.Hkv; g += waves) {
    float* srow = state + ((static_cast<int64_t>(l) * p.R + r) * p.Hkv + g) * p.n_cap;
    if (j0 >= n) {
      // no key of this tile is visible: a region start clears it, later
      // tokens leave the zeros in place (their probability is 0)
      if (t == 0 && j < p.n_cap) srow[j] = 0.f;
      continue;
    }
    const float old = (t > 0) ? srow[jc] : 0.f;
    // A operand: query head `col` of the group, d = 32*ks + 8*qd .. +7
    const bool hv = col < p.G;
    const uint16_t* qrow = static_cast<const uint16_t*>(q) +
                           ((static_cast<int64_t>(l) * p.Ra + a) * p.Hq + g * p.G + (hv ? col : 0)) * D + 8 * qd;
    uint4 qa[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * ks);
      qa[ks] = hv ? v : make_uint4(0u, 0u, 0u, 0u);
    }
    // LSE (log2 units) of the heads this lane's accumulators hold: 4*qd + i
    float lse2[4];
    const float* lrow = lse + (static_cast<int64_t>(l) * p.Ra + a) * p.Hq + g * p.G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * qd + i;
      const float v = lrow[h < p.G ? h : 0];
      lse2[i] = (h < p.G) ? v * kDecLog2e : INFINITY;
    }
    // B operands: key `col` of each sub-page, same d pieces; unmapped or
    // unseen sub-pages read block 0 and are masked afterwards
    uint4 kb[kDecSubPages][KS];
    bool okp[kDecSubPages];
    const int lane_off = col * static_cast<int>(row_elems) + 8 * qd;   // Hkv <= 4096: fits in 32 bits
#pragma unroll
    for (int sp = 0; sp < kDecSubPages; ++sp) {
      const int jp = static_cast<int>(j0) + 16 * sp;    // n_cap <= 2^30
      const int lb = jp / p.block_size;
      const int off = jp - lb * p.block_size;
      const int pb = btab[min(lb, p.Y - 1)];
      okp[sp] = jp < n && pb >= 0 && pb < p.pool_blocks;
      const int64_t pbc = okp[sp] ? pb : 0;
      const uint16_t* kblk = pool + ((static_cast<int64_t>(l) * p.pool_blocks + pbc) * p.block_size + off) * row_elems +
                             static_cast<int64_t>(g) * D;
      const uint16_t* krow = kblk + lane_off;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[sp][ks] = *reinterpret_cast<const uint4*>(krow + 32 * ks);
    }
    float m[kDecSubPages];
#pragma unroll
    for (int sp = 0; sp < kDecSubPages; ++sp) {
      dec_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = dec_mfma<DT>(qa[ks], kb[sp][ks], acc);
      float x = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) x = fmaxf(x, fmaf(acc[i], p.scale2, -lse2[i]));
      if (p.G > 4) {
        x = fmaxf(x, __shfl_xor(x, 16));
        x = fmaxf(x, __shfl_xor(x, 32));
      }
      m[sp] = x;
    }
    // lane -> position j0 + lane: sub-page qd, key col
    float x = -INFINITY;
    bool ok = false;
#pragma unroll
    for (int sp = 0; sp < kDecSubPages; ++sp) {
      const float y = __shfl(m[sp], col);
      if (qd == sp) {
        x = y;
        ok = okp[sp];
      }
    }
    const float prob = (ok && j < n) ? __builtin_amdgcn_exp2f(x) : 0.f;
    if (j < p.n_cap) srow[j] = (t == 0) ? prob : fmaf(prob - old, inv, old);
  }
}

hipError_t launch_decode_score(const DecodeParams& p, int dt, const void* q, const float* lse, const void* k_pool,
                               float* state, hipStream_t st) {
  if (p.Ra == 0 || p.L == 0 || p.n_cap == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(ceil_div(p.n_cap, 64)), p.Ra, p.L);
  const int threads = 64 * min(p.Hkv, 8);
#define KVSEL_DECODE(DTV, DV) decode_score_kernel<DTV, DV><<<grid, threads, 0, st>>>(p, q, lse, k_pool, state)
  if (dt == KVSEL_BF16) {
    if (p.D == 128) KVSEL_DECODE(KVSEL_BF16, 128); else KVSEL_DECODE(KVSEL_BF16, 64);
  } else {
    if (p.D == 128) KVSEL_DECODE(KVSEL_F16, 128); else KVSEL_DECODE(KVSEL_F16, 64);
  }
#undef KVSEL_DECODE
  return hipGetLastError();
}

// ---------------------------------------------------------------- keep score

constexpr int kReduceQuads = 64;    // position quads per block (256 positions, 1 KiB per unit row)
constexpr int kReduceGroups = 4;    // unit groups per block (thread = 64*group + quad)
constexpr int kReduceBatch = 8;     // loads in flight per thread

__device__ __forceinline__ void neumaier_add(double& s, double& c, double v) {
  const double t = s + v;
  c += (fabs(s) >= fabs(v)) ? ((s - t) + v) : ((v - t) + s);
  s = t;
}

// attn[row][j] = float(sum over (l, g) of state[l][r][g][j]), j < n_len[r];
// 0 for n_len[r] <= j < n_cap.  A block covers 256 positions: 64 threads of
// four positions each (1 KiB contiguous per unit row) times 4 groups of
// units; each group keeps a compensated float64 partial and the first wave
// merges the 4 partials in a fixed order.
__global__ __launch_bounds__(256) void action_reduce_kernel(KeepScoreParams p, const float* __restrict__ state,
                                                            float* __restrict__ attn, int attn_by_req) {
  __shared__ double part_s[kReduceGroups][4 * kReduceQuads], part_c[kReduceGroups][4 * kReduceQuads];
  const int a = blockIdx.y;
  const int r = (p.req != nullptr) ? p.req[a] : a;
  if (r < 0 || r >= p.R) return;
  const int64_t n = min(max(static_cast<int64_t>(p.n_len[r]), static_cast<int64_t>(0)), p.n_cap);
  const int quad = threadIdx.x % kReduceQuads, grp = threadIdx.x / kReduceQuads;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 4 * kReduceQuads;
  const int64_t j4 = j0 + 4 * quad;
  float* out = attn + static_cast<int64_t>(attn_by_req ? r : a) * p.n_cap;
  if (j0 >= n) {
    if (grp == 0)
      for (int i = 0; i < 4; ++i)
        if (j4 + i < p.n_cap) out[j4 + i] = 0.f;
    return;
  }
  const int U = p.L * p.Hkv;
  const bool vec = (p.n_cap % 4 == 0) && ((reinterpret_cast<uintptr_t>(state) & 15) == 0) && j4 + 3 < p.n_cap;
  const int64_t jc = min(j4, p.n_cap - 1);
  double s[4] = {0.0, 0.0, 0.0, 0.0}, c[4] = {0.0, 0.0, 0.0, 0.0};
  for (int u0 = grp; u0 < U; u0 += kReduceGroups * kReduceBatch) {
    float4 v[kReduceBatch];
#pragma unroll
    for (int b = 0; b < kReduceBatch; ++b) {
      const int u = min(u0 + kReduceGroups * b, U - 1);
      const int l = u / p.Hkv, g = u - l * p.Hkv;
      const float* src = state + ((static_cast<int64_t>(l) * p.R + r) * p.Hkv + g) * p.n_cap;
      if (vec) {
        v[b] = *reinterpret_cast<const float4*>(src + j4);
      } else {
        v[b].x = src[jc];
        v[b].y = src[min(j4 + 1, p.n_cap - 1)];
        v[b].z = src[min(j4 + 2, p.n_cap - 1)];
        v[b].w = src[min(j4 + 3, p.n_cap - 1)];
      }
    }
#pragma unroll
    for (int b = 0; b < kReduceBatch; ++b) {
      if (u0 + kReduceGroups * b >= U) break;
      neumaier_add(s[0], c[0], static_cast<double>(v[b].x));
      neumaier_add(s[1], c[1], static_cast<double>(v[b].y));
      neumaier_add(s[2], c[2], static_cast<double>(v[b].z));
      neumaier_add(s[3], c[3], static_cast<double>(v[b].w));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    part_s[grp][4 * quad + i] = s[i];
    part_c[grp][4 * quad + i] = c[i];
  }
  __syncthreads();
  if (grp == 0) {
    float res[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double S = 0.0, C = 0.0;
      for (int k = 0; k < kReduceGroups; ++k) {
        neumaier_add(S, C, part_s[k][4 * quad + i]);
        C += part_c[k][4 * quad + i];
      }
      res[i] = (j4 + i < n) ? static_cast<float>(S + C) : 0.f;
    }
    if (vec) {
      *reinterpret_cast<float4*>(out + j4) = make_float4(res[0], res[1], res[2], res[3]);
    } else {
      for (int i = 0; i < 4; ++i)
        if (j4 + i < p.n_cap) out[j4 + i] = res[i];
    }
  }
}

// Ordering bits of a non-negative score (anything not above zero maps to 0).
__device__ __forceinline__ uint32_t weight_key(float v) { return (v > 0.f) ? __float_as_uint(v) : 0u; }

constexpr int kTopPThreads = 1024;

__global__ __launch_bounds__(kTopPThreads) void top_p_update_kernel(KeepScoreParams p, const float* __restrict__ attn,
                                                                    int attn_by_req, float* __restrict__ ks,
                                                                    uint8_t* __restrict__ hit) {
  __shared__ double wsum[256];
  __shared__ uint32_t sh_prefix;
  __shared__ double sh_rem;
  __shared__ int sh_none;
  __shared__ int wave_cnt[kTopPThreads / 64];
  __shared__ int sh_ties;
  const int a = blockIdx.x;
  const int r = (p.req != nullptr) ? p.req[a] : a;
  if (r < 0 || r >= p.R) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = min(max(static_cast<int64_t>(p.n_len[r]), static_cast<int64_t>(0)), p.n_cap);
  const float* row = attn + static_cast<int64_t>(attn_by_req ? r : a) * p.n_cap;
  float* ksr = ks + static_cast<int64_t>(r) * p.n_cap;
  uint8_t* hr = (hit != nullptr) ? hit + static_cast<int64_t>(r) * p.n_cap : nullptr;

  if (tid == 0) {
    sh_prefix = 0u;
    sh_none = 0;
    sh_ties = 0;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) wsum[tid] = 0.0;
    __syncthreads();
    const uint32_t prefix = sh_prefix;
    if (sh_none) break;
    for (int64_t j = tid; j < n; j += kTopPThreads) {
      const float v = row[j];
      const uint32_t key = weight_key(v);
      const bool match = (pass == 0) || ((key >> (shift + 8)) == (prefix >> (shift + 8)));
      if (match && key != 0u) atomicAdd(&wsum[(key >> shift) & 255u], static_cast<double>(v));
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns buckets 255 - 4*lane .. 252 - 4*lane (descending order)
      double w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = wsum[255 - 4 * lane - i];
      const double loc = ((w[0] + w[1]) + w[2]) + w[3];
      // weight above each lane's buckets, accumulated in lane order
      double run = 0.0, above = 0.0;
      for (int k = 0; k < 64; ++k) {
        if (k == lane) above = run;
        run += __shfl(loc, k);
      }
      double rem = (pass == 0) ? static_cast<double>(p.top_p) * run : sh_rem;
      const bool stop = !(rem > 0.0);
      // first bucket (from the top) whose cumulative weight reaches rem, and
      // the lowest non-empty bucket as the fallback when rounding leaves rem
      // above every cumulative weight
      int hit_i = -1, low_i = -1;
      double hit_cum = 0.0, low_cum = 0.0, cb = above;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (w[i] > 0.0) {
          if (hit_i < 0 && cb + w[i] >= rem) {
            hit_i = i;
            hit_cum = cb;
          }
          low_i = i;
          low_cum = cb;
        }
        cb += w[i];
      }
      const uint64_t hits = __ballot(hit_i >= 0), lows = __ballot(low_i >= 0);
      if (!stop && (hits | lows) != 0ull) {
        const bool use_hit = hits != 0ull;
        const int src = use_hit ? (__ffsll(static_cast<long long>(hits)) - 1) : (63 - __clzll(static_cast<long long>(lows)));
        const int bi = __shfl(use_hit ? hit_i : low_i, src);
        const double cum = __shfl(use_hit ? hit_cum : low_cum, src);
        if (lane == 0) {
          sh_prefix = prefix | (static_cast<uint32_t>(255 - 4 * src - bi) << shift);
          sh_rem = rem - cum;
        }
      } else if (lane == 0) {
        sh_none = 1;
      }
    }
    __syncthreads();
  }
  const bool none = sh_none != 0;
  const uint32_t tau = sh_prefix;
  // entries tied at the boundary value join in index order until the
  // remainder is covered
  int64_t c_need = 0;
  if (!none) {
    int cnt = 0;
    for (int64_t j = tid; j < n; j += kTopPThreads) cnt += (weight_key(row[j]) == tau);
    atomicAdd(&sh_ties, cnt);
    __syncthreads();
    const double tv = static_cast<double>(__uint_as_float(tau));
    const double need = ceil(sh_rem / tv);
    c_need = (need < 1.0) ? 1 : (need >= static_cast<double>(sh_ties) ? sh_ties : static_cast<int64_t>(need));
  }
  const bool rank = !none && c_need < sh_ties;
  const float lam = p.lambda;
  int64_t base = 0;   // ties at smaller indices than the current chunk
  for (int64_t j0 = 0; j0 < p.n_cap; j0 += kTopPThreads) {
    const int64_t j = j0 + tid;
    bool h = false;
    uint32_t key = 0u;
    float v = 0.f;
    if (j < n) {
      v = row[j];
      key = weight_key(v);
      h = !none && key > tau;
    }
    const bool tie = !none && j < n && key == tau;
    if (rank && j0 < n) {
      const uint64_t bal = __ballot(tie);
      const int below = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int64_t before = base;
      for (int w = 0; w < wave; ++w) before += wave_cnt[w];
      if (tie && before + below < c_need) h = true;
      int64_t chunk = 0;
      for (int w = 0; w < kTopPThreads / 64; ++w) chunk += wave_cnt[w];
      base += chunk;
      __syncthreads();
    } else if (tie) {
      h = true;
    }
    if (j < n) {
      const float k0 = ksr[j];
      ksr[j] = h ? fmaf(lam, k0, v) : lam * k0;
    }
    if (hr != nullptr && j < p.n_cap) hr[j] = h ? 1 : 0;
  }
}

size_t keep_score_workspace_bytes(const KeepScoreParams& p, bool attn_given) {
  if (attn_given || p.Rc == 0 || p.n_cap == 0) return 0;
  return static_cast<size_t>(p.Rc) * static_cast<size_t>(p.n_cap) * sizeof(float);
}

hipError_t launch_keep_score(const KeepScoreParams& p, const float* state, float* ks, float* attn_out,
                             uint8_t* hit, void* ws, hipStream_t st) {
  if (p.Rc == 0 || p.n_cap == 0) return hipSuccess;
  float* attn = attn_out ? attn_out : static_cast<float*>(ws);
  const int by_req = attn_out != nullptr;
  const dim3 g1(static_cast<unsigned>(ceil_div(p.n_cap, 4 * kReduceQuads)), p.Rc);
  action_reduce_kernel<<<g1, 256, 0, st>>>(p, state, attn, by_req);
  top_p_update_kernel<<<p.Rc, kTopPThreads, 0, st>>>(p, attn, by_req, ks, hit);
  return hipGetLastError();
}

}  // namespace kvsel
