// Token-level window scores: softmax of a query window against every cached
// key, aggregated over the GQA group and the window rows.
//
// ActKV §2: the score of a cached key is its attention weight
// softmax(q.k / sqrt(D)).  ActKV §7.1: the weights are recovered as
// exp(s - LSE) from the log-sum-exp of each query row, so a score pass only
// needs the LSE and fresh q.k products.  Two passes therefore: the LSE of
// every window row (unless the caller supplies it), then the recovered
// probabilities summed per key.
//
// MFMA path (bf16/f16, D in {64, 128}, W >= 16, G*W <= 256): one workgroup
// per (unit, chunk of keys), one wavefront per 64 query rows held in
// registers as MFMA operands; 64-key tiles of K are staged through LDS
// (double buffered, padded rows) and contracted with
// v_mfma_f32_32x32x16.  The score pass keeps keys on the MFMA output's
// column axis so the sum over query rows is a per-lane register sum plus
// one cross-half shuffle; the LSE pass swaps the operands so each lane owns
// one query row and keeps an online max/sum in registers.
//
// VALU path: any dtype/shape/aggregation, one lane per key (the LSE pass:
// one wavefront per chunk of keys, merged like the matrix-core partials).
#include "common.h"

#include <math.h>
#include <climits>

namespace kvsel {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
}  // namespace

// =================================================================== VALU path

// 16 bytes of a row as floats (4 of F32, 8 of BF16/F16).
template <int DT>
__device__ __forceinline__ void load16_floats(const void* base, int64_t elem, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + elem * (DT == KVSEL_F32 ? 4 : 2));
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == KVSEL_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t lo = static_cast<uint16_t>(w[i] & 0xFFFFu), hi = static_cast<uint16_t>(w[i] >> 16);
      out[2 * i] = (DT == KVSEL_BF16) ? bf16_to_f32(lo) : f16_to_f32(lo);
      out[2 * i + 1] = (DT == KVSEL_BF16) ? bf16_to_f32(hi) : f16_to_f32(hi);
    }
  }
}

// LSE pass: one wavefront per (chunk of keys, group of kRowGroup query
// rows, unit).  The group's rows sit in LDS as floats; each lane owns keys
// lane, lane + 64, ... of the chunk (its K row read with 16-byte loads) and
// keeps an online max/sum of exp2(c1 * q.k) per row.  The wavefront's
// (max, sum) per row, reduced in a fixed order, go to the partials that
// lse_combine_kernel merges, as in the matrix-core path.  Short wavefronts
// keep the dependent chain of each one short: small windows run on few
// keys, where latency, not throughput, sets the time.
constexpr int kLseValuRowGroup = 4;

template <int DT, int D>
__global__ __launch_bounds__(64) void lse_valu_kernel(WindowParams p, const void* __restrict__ q,
                                                      const void* __restrict__ k, int chunk_keys,
                                                      float2* __restrict__ partials) {
  __shared__ float qs[kLseValuRowGroup * D];
  constexpr int E = (DT == KVSEL_F32) ? 4 : 8;
  const int u = blockIdx.z, chunk = blockIdx.x, n_chunks = gridDim.x;
  const int r0 = blockIdx.y * kLseValuRowGroup;
  const int lane = threadIdx.x;
  const int l = u / p.Hkv, g = u % p.Hkv;
  const int R = p.G * p.W;
  for (int e = lane; e < kLseValuRowGroup * D; e += 64) {
    const int r = r0 + e / D, d = e % D;
    const int h = g * p.G + r / p.W, t = r % p.W;
    qs[e] = (r < R) ? load_elem<DT>(q, ((static_cast<int64_t>(l) * p.Hq + h) * p.W + t) * D + d) : 0.f;
  }
  __syncthreads();
  const int64_t key0 = static_cast<int64_t>(chunk) * chunk_keys;
  const int64_t key1 = min(p.N, key0 + chunk_keys);
  const int64_t kb = (static_cast<int64_t>(l) * p.Hkv + g) * p.N * D;
  const float c1 = p.scale * kLog2e;
  {
    float m[kLseValuRowGroup], s[kLseValuRowGroup];
#pragma unroll
    for (int i = 0; i < kLseValuRowGroup; ++i) {
      m[i] = -INFINITY;
      s[i] = 0.f;
    }
    for (int64_t j = key0 + lane; j < key1; j += 64) {
      float kr[D];
#pragma unroll
      for (int d = 0; d < D; d += E) load16_floats<DT>(k, kb + j * D + d, kr + d);
#pragma unroll
      for (int i = 0; i < kLseValuRowGroup; ++i) {
        const int r = r0 + i;
        if (r < R && (!p.causal || j <= p.N - p.W + r % p.W)) {
          const float* qr = qs + i * D;
          float acc = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) acc = fmaf(qr[d], kr[d], acc);
          const float x = acc * c1;
          if (x > m[i]) {
            s[i] = s[i] * exp2f(m[i] - x) + 1.f;
            m[i] = x;
          } else {
            s[i] += exp2f(x - m[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kLseValuRowGroup; ++i) {
      float mm = m[i], ss = s[i];
      for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(mm, o, 64);
        const float s2 = __shfl_xor(ss, o, 64);
        const float mn = fmaxf(mm, m2);
        const float a = (mm == -INFINITY) ? 0.f : ss * exp2f(mm - mn);
        const float b = (m2 == -INFINITY) ? 0.f : s2 * exp2f(m2 - mn);
        mm = mn;
        ss = a + b;
      }
      if (lane == 0 && r0 + i < R)
        partials[(static_cast<int64_t>(u) * n_chunks + chunk) * R + r0 + i] = make_float2(mm, ss);
    }
  }
}

// One row's LSE (natural log) from its chunks' (max, sum) partials (log2
// domain, chunk c at pr[c * stride]): merged online in chunk order, eight
// loads in flight at a time.  The combine kernel and the fused score-pass
// prologue both call this, so the value has the same bits either way.
__device__ __forceinline__ float merge_row_partials(const float2* __restrict__ pr, int n_chunks, int stride) {
  constexpr int kBatch = 8;
  float m = -INFINITY, s = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += kBatch) {
    float2 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      v[j] = (c0 + j < n_chunks) ? pr[static_cast<int64_t>(c0 + j) * stride] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (v[j].x == -INFINITY) continue;
      const float mn = fmaxf(m, v[j].x);
      s = ((m == -INFINITY) ? 0.f : s * exp2f(m - mn)) + v[j].y * exp2f(v[j].x - mn);
      m = mn;
    }
  }
  return (m + log2f(s)) * kLn2;
}

// Score pass: a workgroup per (64 keys, unit), one key per lane; its four
// wavefronts split the window rows (wavefront w takes rows t = w, w + 4, ...)
// and their per-key row aggregates are combined in wavefront order through
// LDS, so each lane's dependent chain is a quarter of the window.  With the
// LSE pass's chunk partials given (when the caller wants no LSE
// output, `lse_part`), each workgroup merges its unit's rows itself instead
// of reading `lse`, which saves the combine launch.
template <int DT, int D>
__global__ __launch_bounds__(256) void scores_valu_kernel(WindowParams p, const void* __restrict__ q,
                                                          const void* __restrict__ k,
                                                          const float* __restrict__ lse,
                                                          const float2* __restrict__ lse_part, int n_chunks,
                                                          float* __restrict__ out) {
  extern __shared__ float sm[];          // [G*W][D] queries, then [G*W] lse
  __shared__ float part[4][64];
  constexpr int E = (DT == KVSEL_F32) ? 4 : 8;
  const int u = blockIdx.y;
  const int l = u / p.Hkv, g = u % p.Hkv;
  const int R = p.G * p.W;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float* qs = sm;
  float* ls = sm + static_cast<int64_t>(R) * D;
  for (int64_t e = threadIdx.x; e < static_cast<int64_t>(R) * D; e += blockDim.x) {
    const int r = static_cast<int>(e / D), d = static_cast<int>(e % D);
    const int h = g * p.G + r / p.W, t = r % p.W;
    qs[e] = load_elem<DT>(q, ((static_cast<int64_t>(l) * p.Hq + h) * p.W + t) * D + d);
  }
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int h = g * p.G + r / p.W, t = r % p.W;
    ls[r] = (lse_part != nullptr)
                ? merge_row_partials(lse_part + static_cast<int64_t>(u) * n_chunks * R + r, n_chunks, R)
                : lse[(static_cast<int64_t>(l) * p.Hq + h) * p.W + t];
  }
  __syncthreads();
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool valid = j < p.N;
  float kr[D];
  const int64_t kb = ((static_cast<int64_t>(l) * p.Hkv + g) * p.N + (valid ? j : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; d += E) load16_floats<DT>(k, kb + d, kr + d);
  const bool rmax = p.row_agg == KVSEL_AGG_MAX;
  float racc = 0.f;
  for (int t = w; t < p.W; t += 4) {
    const bool allowed = !p.causal || j <= p.N - p.W + t;
    float hacc = 0.f;
    for (int hl = 0; hl < p.G; ++hl) {
      const int r = hl * p.W + t;
      float pr = 0.f;
      if (allowed) {
        float acc = 0.f;
        const float* qr = qs + static_cast<int64_t>(r) * D;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(qr[d], kr[d], acc);
        pr = expf(acc * p.scale - ls[r]);
      }
      hacc = (p.head_agg == KVSEL_AGG_MAX) ? fmaxf(hacc, pr) : hacc + pr;
    }
    if (p.head_agg == KVSEL_AGG_MEAN) hacc /= static_cast<float>(p.G);
    racc = rmax ? fmaxf(racc, hacc) : racc + hacc;
  }
  part[w][lane] = racc;
  __syncthreads();
  if (w != 0 || !valid) return;
  float tot = part[0][lane];
#pragma unroll
  for (int x = 1; x < 4; ++x) tot = rmax ? fmaxf(tot, part[x][lane]) : tot + part[x][lane];
  if (p.row_agg == KVSEL_AGG_MEAN) tot /= static_cast<float>(p.W);
  out[static_cast<int64_t>(u) * p.N + j] = tot;
}

template <int DT, int D>
static hipError_t launch_scores_valu_t(const WindowParams& p, const void* q, const void* k,
                                       const float* lse, const float2* part, int n_chunks, float* out,
                                       hipStream_t st) {
  const size_t sh = (static_cast<size_t>(p.G) * p.W * D + static_cast<size_t>(p.G) * p.W) * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scores_valu_kernel<DT, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(sh));
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>(ceil_div(p.N, 64)), static_cast<unsigned>(p.L * p.Hkv));
  scores_valu_kernel<DT, D><<<grid, 256, sh, st>>>(p, q, k, lse, part, n_chunks, out);
  return hipGetLastError();
}

static int lse_valu_chunk_keys(const WindowParams& p);

hipError_t launch_window_scores_valu(const WindowParams& p, int dt, const void* q, const void* k,
                                     const float* lse, const float* partials, float* out, hipStream_t st) {
  if (p.N == 0 || p.L * p.Hkv == 0) return hipSuccess;
  const float2* part = reinterpret_cast<const float2*>(partials);
  const int n_chunks = static_cast<int>(ceil_div(p.N, lse_valu_chunk_keys(p)));
#define KVSEL_SV(DTV)                                                                   \
  return (p.D == 64) ? launch_scores_valu_t<DTV, 64>(p, q, k, lse, part, n_chunks, out, st) \
                     : launch_scores_valu_t<DTV, 128>(p, q, k, lse, part, n_chunks, out, st)
  if (dt == KVSEL_F32) { KVSEL_SV(KVSEL_F32); }
  if (dt == KVSEL_BF16) { KVSEL_SV(KVSEL_BF16); }
  KVSEL_SV(KVSEL_F16);
#undef KVSEL_SV
}

// =================================================================== MFMA path

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileKeys = 64;          // keys per LDS tile (two 32-wide MFMA column blocks)
constexpr int kChunkKeys = 2048;       // keys per workgroup

template <int DT>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (DT == KVSEL_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Shared layout of both MFMA kernels.
template <int D>
struct MfmaTile {
  static constexpr int kRowBytes = D * 2 + 16;                 // padded K row in LDS
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
  static constexpr int kKSteps = D / 16;                       // MFMA k-steps per dot product
  static constexpr int kChunksPerRow = D * 2 / 16;             // 16-byte pieces per K row
  static constexpr int kLoadsPerThread = kTileKeys * kChunksPerRow / 256;
};

// Query operand fragments of this wavefront's 64 rows.  Lane l holds, for row
// block rb and k-step ks, the 8 elements d = 16*ks + 8*(l/32) .. +7 of row
// 64*w + 32*rb + l%32.  The same registers serve as the A operand (rows on
// the output's row axis) and as the B operand (rows on the column axis).
template <int DT, int D>
__device__ __forceinline__ void load_q_frags(const WindowParams& p, const void* q, int l, int g,
                                             int wave, int lane, uint4 (&qf)[2][D / 16]) {
  const int R = p.G * p.W;
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 64 * wave + 32 * rb + (lane & 31);
    const bool ok = r < R;
    const int h = g * p.G + (ok ? r / p.W : 0), t = ok ? r % p.W : 0;
    const uint8_t* src = static_cast<const uint8_t*>(q) +
                         (((static_cast<int64_t>(l) * p.Hq + h) * p.W + t) * D) * 2;
    for (int ks = 0; ks < D / 16; ++ks) {
      const int d = 16 * ks + 8 * (lane >> 5);
      qf[rb][ks] = ok ? *reinterpret_cast<const uint4*>(src + d * 2) : make_uint4(0, 0, 0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_k_tile_regs(const uint8_t* kunit, int64_t key0, int64_t N,
                                                 uint4 (&reg)[MfmaTile<D>::kLoadsPerThread]) {
  using T = MfmaTile<D>;
  for (int i = 0; i < T::kLoadsPerThread; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int key = c / T::kChunksPerRow, piece = c % T::kChunksPerRow;
    const int64_t j = key0 + key;
    reg[i] = (j < N) ? *reinterpret_cast<const uint4*>(kunit + (j * D) * 2 + piece * 16)
                     : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_k_tile_lds(uint8_t* buf,
                                                 const uint4 (&reg)[MfmaTile<D>::kLoadsPerThread]) {
  using T = MfmaTile<D>;
  for (int i = 0; i < T::kLoadsPerThread; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int key = c / T::kChunksPerRow, piece = c % T::kChunksPerRow;
    *reinterpret_cast<uint4*>(buf + key * T::kRowBytes + piece * 16) = reg[i];
  }
}

// K operand fragment: key 32*cb + l%32 of the tile, elements d = 16*ks + 8*(l/32) ..
template <int D>
__device__ __forceinline__ uint4 k_frag(const uint8_t* buf, int cb, int ks, int lane) {
  using T = MfmaTile<D>;
  const int key = 32 * cb + (lane & 31);
  const int d = 16 * ks + 8 * (lane >> 5);
  return *reinterpret_cast<const uint4*>(buf + key * T::kRowBytes + d * 2);
}

}  // namespace

// ---- pass 1: per-(unit, chunk) partial (max, sum) of every row, log2 domain
// Tiles whose keys every row may see take a branch-free path; only the
// causal tail and the ragged end check keys one by one.  K streams through
// the same three register staging sets as the score pass.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DeepStage {
  static constexpr int kN = MfmaTile<D>::kLoadsPerThread;        // 16-byte pieces per thread
  u32x4 r[kN];
};

template <int D>
__device__ __forceinline__ void deep_load(const uint8_t* kunit, int key0, int N, DeepStage<D>& st) {
  using T = MfmaTile<D>;
#pragma unroll
  for (int i = 0; i < DeepStage<D>::kN; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int j = min(key0 + c / T::kChunksPerRow, N - 1);
    st.r[i] = *reinterpret_cast<const u32x4*>(kunit + static_cast<int64_t>(j) * (D * 2) + (c % T::kChunksPerRow) * 16);
  }
}

template <int D>
__device__ __forceinline__ void deep_store(uint8_t* buf, const DeepStage<D>& st) {
  using T = MfmaTile<D>;
#pragma unroll
  for (int i = 0; i < DeepStage<D>::kN; ++i) {
    const int c = threadIdx.x + 256 * i;
    *reinterpret_cast<u32x4*>(buf + (c / T::kChunksPerRow) * T::kRowBytes + (c % T::kChunksPerRow) * 16) = st.r[i];
  }
}

#define KVSEL_LSE_TILE(TI, SET)                                                                  \
  do {                                                                                           \
    const int ti_ = (TI);                                                                        \
    if (ti_ < n_tiles) {                                                                         \
      const int key0 = key_begin + ti_ * kTileKeys;                                              \
      const uint8_t* buf = kbuf[ti_ & 1];                                                        \
      f32x16 acc[2][2];                                                                          \
      for (int cb = 0; cb < 2; ++cb)                                                             \
        for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = f32x16{};                                   \
      for (int ks = 0; ks < T::kKSteps; ++ks) {                                                  \
        const uint4 kf0 = k_frag<D>(buf, 0, ks, lane);                                           \
        const uint4 kf1 = k_frag<D>(buf, 1, ks, lane);                                           \
        for (int rb = 0; rb < 2; ++rb) {                                                         \
          acc[0][rb] = mfma32<DT>(kf0, qf[rb][ks], acc[0][rb]);                                  \
          acc[1][rb] = mfma32<DT>(kf1, qf[rb][ks], acc[1][rb]);                                  \
        }                                                                                        \
      }                                                                                          \
      const bool full = key0 + kTileKeys <= min(first_masked, key_end);                          \
      const int kl = key0 + 4 * (lane >> 5);                                                     \
      for (int rb = 0; rb < 2; ++rb) {                                                           \
        if (lim[rb] < 0) continue;                                                               \
        float tmax = -INFINITY;                                                                  \
        if (full) {                                                                              \
          for (int cb = 0; cb < 2; ++cb)                                                         \
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, acc[cb][rb][v]);                     \
        } else {                                                                                 \
          for (int cb = 0; cb < 2; ++cb)                                                         \
            for (int v = 0; v < 16; ++v) {                                                       \
              const int key = kl + 32 * cb + 8 * (v >> 2) + (v & 3);                             \
              if (key <= lim[rb] && key < key_end) tmax = fmaxf(tmax, acc[cb][rb][v]);           \
            }                                                                                    \
          if (tmax == -INFINITY) continue;                                                       \
        }                                                                                        \
        const float mn = fmaxf(m[rb], tmax * c1);                                                \
        float sum = 0.f;                                                                         \
        if (full) {                                                                              \
          for (int cb = 0; cb < 2; ++cb)                                                         \
            for (int v = 0; v < 16; ++v)                                                         \
              sum += __builtin_amdgcn_exp2f(fmaf(acc[cb][rb][v], c1, -mn));                      \
        } else {                                                                                 \
          for (int cb = 0; cb < 2; ++cb)                                                         \
            for (int v = 0; v < 16; ++v) {                                                       \
              const int key = kl + 32 * cb + 8 * (v >> 2) + (v & 3);                             \
              const float e = __builtin_amdgcn_exp2f(fmaf(acc[cb][rb][v], c1, -mn));             \
              sum += (key <= lim[rb] && key < key_end) ? e : 0.f;                                \
            }                                                                                    \
        }                                                                                        \
        s[rb] = s[rb] * __builtin_amdgcn_exp2f(m[rb] - mn) + sum;                                \
        m[rb] = mn;                                                                              \
      }                                                                                          \
    }                                                                                            \
    deep_store<D>(kbuf[(ti_ + 1) & 1], SET);                                                     \
    deep_load<D>(kunit, key_begin + min(ti_ + 4, n_tiles - 1) * kTileKeys, N, SET);              \
    __syncthreads();                                                                             \
  } while (0)

template <int DT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lse_mfma_kernel(WindowParams p, const void* __restrict__ q, const void* __restrict__ k,
                     float2* __restrict__ partials) {
  using T = MfmaTile<D>;
  __shared__ __align__(16) uint8_t kbuf[2][T::kTileBytes];
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int l = u / p.Hkv, g = u % p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.G * p.W;
  const int N = static_cast<int>(p.N);
  const int key_begin = chunk * kChunkKeys;
  const int key_end = min(N, key_begin + kChunkKeys);
  const uint8_t* kunit = static_cast<const uint8_t*>(k) +
                         ((static_cast<int64_t>(l) * p.Hkv + g) * p.N * D) * 2;
  const int n_tiles = (key_end - key_begin + kTileKeys - 1) / kTileKeys;
  uint4 qf[2][D / 16];
  load_q_frags<DT, D>(p, q, l, g, wave, lane, qf);
  const float c1 = p.scale * kLog2e;
  int lim[2];                       // last key each of this lane's two rows may see
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 64 * wave + 32 * rb + (lane & 31);
    lim[rb] = (r >= R) ? -1 : (p.causal ? N - p.W + r % p.W : N - 1);
  }
  const int first_masked = p.causal ? N - p.W + 1 : N;
  float m[2] = {-INFINITY, -INFINITY}, s[2] = {0.f, 0.f};
  // the K prefetches are issued after the query loads; tile t waits in set t % 3
  DeepStage<D> s0, s1, s2;
  deep_load<D>(kunit, key_begin, N, s0);
  deep_load<D>(kunit, key_begin + min(1, n_tiles - 1) * kTileKeys, N, s1);
  deep_load<D>(kunit, key_begin + min(2, n_tiles - 1) * kTileKeys, N, s2);
  deep_store<D>(kbuf[0], s0);
  deep_load<D>(kunit, key_begin + min(3, n_tiles - 1) * kTileKeys, N, s0);
  __syncthreads();
  for (int ti = 0; ti < n_tiles; ti += 3) {
    KVSEL_LSE_TILE(ti, s1);
    KVSEL_LSE_TILE(ti + 1, s2);
    KVSEL_LSE_TILE(ti + 2, s0);
  }
  // combine the two lane halves (they hold the other half of each tile's keys)
  for (int rb = 0; rb < 2; ++rb) {
    const float m2 = __shfl_xor(m[rb], 32, 64);
    const float s2v = __shfl_xor(s[rb], 32, 64);
    const float mn = fmaxf(m[rb], m2);
    const float a = (m[rb] == -INFINITY) ? 0.f : s[rb] * __builtin_amdgcn_exp2f(m[rb] - mn);
    const float b = (m2 == -INFINITY) ? 0.f : s2v * __builtin_amdgcn_exp2f(m2 - mn);
    const int r = 64 * wave + 32 * rb + (lane & 31);
    if (lane < 32 && r < R) {
      const int64_t o = (static_cast<int64_t>(u) * gridDim.x + chunk) * R + r;
      partials[o] = make_float2(mn, a + b);
    }
  }
}
#undef KVSEL_LSE_TILE

// ---- combine chunk partials into LSE [L][Hq][W] (natural log)
// One thread per query row (adjacent rows read adjacent partials): the
// chunks' (max, sum) pairs (log2 domain) merged online in chunk order, eight
// loads in flight at a time; the row's LSE in natural-log units.
__global__ __launch_bounds__(256) void lse_combine_kernel(WindowParams p, int n_chunks,
                                                          const float2* __restrict__ partials,
                                                          float* __restrict__ lse) {
  const int R = p.G * p.W;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = static_cast<int64_t>(p.L) * p.Hkv * R;
  if (i >= n) return;
  const int64_t u = i / R;
  const int r = static_cast<int>(i % R);
  const int l = static_cast<int>(u / p.Hkv), g = static_cast<int>(u % p.Hkv);
  const int h = g * p.G + r / p.W, t = r % p.W;
  lse[(static_cast<int64_t>(l) * p.Hq + h) * p.W + t] = merge_row_partials(partials + u * n_chunks * R + r, n_chunks, R);
}

// ---- pass 2: recovered probabilities summed over the unit's rows, per key
// Three register staging sets keep three 64-key tiles in flight from HBM per
// workgroup on top of the two LDS tile buffers.  Column sums collect in LDS
// and leave in one coalesced store after the last K load, so no global store
// sits between the prefetches; every load is issued unconditionally (past
// the end it re-reads the last tile) so the wait counts stay exact.
#define KVSEL_SC_TILE(TI, SET)                                                                   \
  do {                                                                                           \
    const int ti_ = (TI);                                                                        \
    if (ti_ < n_tiles) {                                                                         \
      const int key0 = key_begin + ti_ * kTileKeys;                                              \
      const uint8_t* buf = kbuf[ti_ & 1];                                                        \
      const bool full = key0 + kTileKeys <= min(first_masked, key_end);                          \
      for (int cb = 0; cb < 2; ++cb) {                                                           \
        f32x16 acc[2];                                                                           \
        acc[0] = f32x16{};                                                                       \
        acc[1] = f32x16{};                                                                       \
        for (int ks = 0; ks < T::kKSteps; ++ks) {                                                \
          const uint4 kf = k_frag<D>(buf, cb, ks, lane);                                         \
          acc[0] = mfma32<DT>(qf[0][ks], kf, acc[0]);                                            \
          acc[1] = mfma32<DT>(qf[1][ks], kf, acc[1]);                                            \
        }                                                                                        \
        const int key = key0 + 32 * cb + (lane & 31);                                            \
        const int kk = key < key_end ? key : INT_MAX;                                            \
        float sum = 0.f;                                                                         \
        if (full) {                                                                              \
          for (int rb = 0; rb < 2; ++rb)                                                         \
            for (int g4 = 0; g4 < 4; ++g4) {                                                     \
              const int r0 = 64 * wave + 32 * rb + 8 * g4 + 4 * (lane >> 5);                     \
              const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[r0]);                    \
              sum += __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 0], c1, -l4.x));               \
              sum += __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 1], c1, -l4.y));               \
              sum += __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 2], c1, -l4.z));               \
              sum += __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 3], c1, -l4.w));               \
            }                                                                                    \
        } else {                                                                                 \
          for (int rb = 0; rb < 2; ++rb)                                                         \
            for (int g4 = 0; g4 < 4; ++g4) {                                                     \
              const int r0 = 64 * wave + 32 * rb + 8 * g4 + 4 * (lane >> 5);                     \
              const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[r0]);                    \
              const int4 m4 = *reinterpret_cast<const int4*>(&lim_s[r0]);                        \
              const float e0 = __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 0], c1, -l4.x));    \
              const float e1 = __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 1], c1, -l4.y));    \
              const float e2 = __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 2], c1, -l4.z));    \
              const float e3 = __builtin_amdgcn_exp2f(fmaf(acc[rb][4 * g4 + 3], c1, -l4.w));    \
              sum += kk <= m4.x ? e0 : 0.f;                                                      \
              sum += kk <= m4.y ? e1 : 0.f;                                                      \
              sum += kk <= m4.z ? e2 : 0.f;                                                      \
              sum += kk <= m4.w ? e3 : 0.f;                                                      \
            }                                                                                    \
        }                                                                                        \
        sum += __shfl_xor(sum, 32, 64);                                                          \
        if (lane < 32) red[ti_ & 1][wave][32 * cb + lane] = sum;                                 \
      }                                                                                          \
    }                                                                                            \
    deep_store<D>(kbuf[(ti_ + 1) & 1], SET);                                                     \
    deep_load<D>(kunit, key_begin + min(ti_ + 2 + 1, n_tiles - 1) * kTileKeys, N, SET);       \
    __syncthreads();                                                                             \
    if (ti_ < n_tiles && threadIdx.x < kTileKeys) {                                              \
      outbuf[ti_ * kTileKeys + threadIdx.x] =                                                    \
          (red[ti_ & 1][0][threadIdx.x] + red[ti_ & 1][1][threadIdx.x] +                         \
           red[ti_ & 1][2][threadIdx.x] + red[ti_ & 1][3][threadIdx.x]) * factor;                \
    }                                                                                            \
  } while (0)

template <int DT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void scores_mfma_kernel(WindowParams p, const void* __restrict__ q, const void* __restrict__ k,
                        const float* __restrict__ lse, float* __restrict__ out) {
  using T = MfmaTile<D>;
  __shared__ __align__(16) uint8_t kbuf[2][T::kTileBytes];
  __shared__ float red[2][4][kTileKeys];
  __shared__ __align__(16) float lse_s[256];
  __shared__ __align__(16) int lim_s[256];      // last key each row may see (-1: no row)
  __shared__ __align__(16) float outbuf[kChunkKeys];
  const int u = blockIdx.y, chunk = blockIdx.x;
  const int l = u / p.Hkv, g = u % p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.G * p.W;
  const int N = static_cast<int>(p.N);
  const int key_begin = chunk * kChunkKeys;
  const int key_end = min(N, key_begin + kChunkKeys);
  const uint8_t* kunit = static_cast<const uint8_t*>(k) +
                         ((static_cast<int64_t>(l) * p.Hkv + g) * p.N * D) * 2;
  const int n_tiles = (key_end - key_begin + kTileKeys - 1) / kTileKeys;
  uint4 qf[2][D / 16];
  load_q_frags<DT, D>(p, q, l, g, wave, lane, qf);
  const float c1 = p.scale * kLog2e;
  {
    const int r = threadIdx.x;                   // 256 threads, one row each
    const bool ok = r < R;
    const int h = g * p.G + (ok ? r / p.W : 0), t = ok ? r % p.W : 0;
    lse_s[r] = ok ? lse[(static_cast<int64_t>(l) * p.Hq + h) * p.W + t] * kLog2e : INFINITY;
    lim_s[r] = !ok ? -1 : p.causal ? N - p.W + t : N - 1;
  }
  // the K prefetches are issued after every other load, so waiting for a
  // tile never waits for more than the loads in front of it
  DeepStage<D> s0, s1;
  deep_load<D>(kunit, key_begin, N, s0);
  deep_load<D>(kunit, key_begin + min(1, n_tiles - 1) * kTileKeys, N, s1);
  float factor = 1.f;
  if (p.head_agg == KVSEL_AGG_MEAN) factor /= static_cast<float>(p.G);
  if (p.row_agg == KVSEL_AGG_MEAN) factor /= static_cast<float>(p.W);
  const int first_masked = p.causal ? N - p.W + 1 : N;   // keys >= this need a per-row check
  deep_store<D>(kbuf[0], s0);
  deep_load<D>(kunit, key_begin + min(2, n_tiles - 1) * kTileKeys, N, s0);
  __syncthreads();
  for (int ti = 0; ti < n_tiles; ti += 2) {
    KVSEL_SC_TILE(ti, s1);
    KVSEL_SC_TILE(ti + 1, s0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < key_end - key_begin; i += 256)
    out[static_cast<int64_t>(u) * p.N + key_begin + i] = outbuf[i];
}
#undef KVSEL_SC_TILE

bool window_mfma_supported(const WindowParams& p, int dt) {
  const int R = p.G * p.W;
  return (dt == KVSEL_BF16 || dt == KVSEL_F16) && (p.D == 64 || p.D == 128) && p.W >= 16 &&
         R <= 256 && p.head_agg != KVSEL_AGG_MAX && p.row_agg != KVSEL_AGG_MAX;
}

size_t window_mfma_partials_bytes(const WindowParams& p) {
  const int64_t n_chunks = ceil_div(p.N, kChunkKeys);
  return static_cast<size_t>(p.L) * p.Hkv * n_chunks * p.G * p.W * sizeof(float2);
}

hipError_t launch_window_lse_mfma(const WindowParams& p, int dt, const void* q, const void* k,
                                  float* partials, float* lse, hipStream_t st) {
  const int n_chunks = static_cast<int>(ceil_div(p.N, kChunkKeys));
  const int U = p.L * p.Hkv;
  if (n_chunks == 0 || U == 0) return hipSuccess;
  const int threads = 256;   // one wavefront per 64 rows; rows >= G*W are masked
  dim3 grid(n_chunks, U);
  float2* part = reinterpret_cast<float2*>(partials);
#define KVSEL_LM(DTV, DV) lse_mfma_kernel<DTV, DV><<<grid, threads, 0, st>>>(p, q, k, part)
  if (dt == KVSEL_BF16) {
    if (p.D == 64) KVSEL_LM(KVSEL_BF16, 64); else KVSEL_LM(KVSEL_BF16, 128);
  } else {
    if (p.D == 64) KVSEL_LM(KVSEL_F16, 64); else KVSEL_LM(KVSEL_F16, 128);
  }
#undef KVSEL_LM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(U) * p.G * p.W;
  lse_combine_kernel<<<static_cast<int>(ceil_div(n, 256)), 256, 0, st>>>(p, n_chunks, part, lse);
  return hipGetLastError();
}

// Keys per wavefront of the VALU LSE pass: 64, or more so that there are at
// most 256 chunks per unit.
static int lse_valu_chunk_keys(const WindowParams& p) {
  const int64_t c = ceil_div(ceil_div(p.N, 256), 64) * 64;
  return static_cast<int>(max(static_cast<int64_t>(64), c));
}

size_t window_valu_partials_bytes(const WindowParams& p) {
  const int64_t n_chunks = ceil_div(p.N, lse_valu_chunk_keys(p));
  return static_cast<size_t>(p.L) * p.Hkv * n_chunks * p.G * p.W * sizeof(float2);
}

template <int DT, int D>
static hipError_t launch_lse_valu_t(const WindowParams& p, const void* q, const void* k, float2* part,
                                    float* lse, hipStream_t st) {
  // lse == nullptr: the partials only (the score pass merges them)
  const int ck = lse_valu_chunk_keys(p);
  const int n_chunks = static_cast<int>(ceil_div(p.N, ck));
  const int U = p.L * p.Hkv;
  const int groups = static_cast<int>(ceil_div(static_cast<int64_t>(p.G) * p.W, kLseValuRowGroup));
  lse_valu_kernel<DT, D><<<dim3(n_chunks, groups, U), 64, 0, st>>>(p, q, k, ck, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || lse == nullptr) return e;
  const int64_t n = static_cast<int64_t>(U) * p.G * p.W;
  lse_combine_kernel<<<static_cast<int>(ceil_div(n, 256)), 256, 0, st>>>(p, n_chunks, part, lse);
  return hipGetLastError();
}

hipError_t launch_window_lse_valu(const WindowParams& p, int dt, const void* q, const void* k,
                                  float* partials, float* lse, hipStream_t st) {
  if (p.N == 0 || p.L * p.Hkv == 0) return hipSuccess;
  float2* part = reinterpret_cast<float2*>(partials);
#define KVSEL_LV(DTV)                                                                   \
  return (p.D == 64) ? launch_lse_valu_t<DTV, 64>(p, q, k, part, lse, st)               \
                     : launch_lse_valu_t<DTV, 128>(p, q, k, part, lse, st)
  if (dt == KVSEL_F32) { KVSEL_LV(KVSEL_F32); }
  if (dt == KVSEL_BF16) { KVSEL_LV(KVSEL_BF16); }
  KVSEL_LV(KVSEL_F16);
#undef KVSEL_LV
}

hipError_t launch_window_scores_mfma(const WindowParams& p, int dt, const void* q, const void* k,
                                     const float* lse, float* out, hipStream_t st) {
  const int n_chunks = static_cast<int>(ceil_div(p.N, kChunkKeys));
  const int U = p.L * p.Hkv;
  if (n_chunks == 0 || U == 0) return hipSuccess;
  const int threads = 256;
  dim3 grid(n_chunks, U);
#define KVSEL_SM(DTV, DV) scores_mfma_kernel<DTV, DV><<<grid, threads, 0, st>>>(p, q, k, lse, out)
  if (dt == KVSEL_BF16) {
    if (p.D == 64) KVSEL_SM(KVSEL_BF16, 64); else KVSEL_SM(KVSEL_BF16, 128);
  } else {
    if (p.D == 64) KVSEL_SM(KVSEL_F16, 64); else KVSEL_SM(KVSEL_F16, 128);
  }
#undef KVSEL_SM
  return hipGetLastError();
}

// =================================================================== pooling

__global__ void pool1d_kernel(const float* __restrict__ in, float* __restrict__ out, int64_t rows,
                              int64_t n, int kind, int ksize) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n, j = i % n;
  const float* row = in + r * n;
  const int h = ksize / 2;
  float acc = (kind == KVSEL_POOL_MAX) ? -INFINITY : 0.f;
  for (int o = -h; o <= h; ++o) {
    const int64_t jj = j + o;
    if (jj < 0 || jj >= n) continue;
    acc = (kind == KVSEL_POOL_MAX) ? fmaxf(acc, row[jj]) : acc + row[jj];
  }
  out[i] = (kind == KVSEL_POOL_MAX) ? acc : acc / static_cast<float>(ksize);
}

hipError_t launch_pool1d(const float* in, float* out, int64_t rows, int64_t n, int kind, int ksize,
                         hipStream_t st) {
  const int64_t total = rows * n;
  if (total == 0) return hipSuccess;
  pool1d_kernel<<<static_cast<int>(ceil_div(total, 256)), 256, 0, st>>>(in, out, rows, n, kind, ksize);
  return hipGetLastError();
}

}  // namespace kvsel
