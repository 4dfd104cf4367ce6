// Block scores against a RoPE-stripped Mean-K index.
//
// KVMem (query-conditioned retrieval): one Mean-K vector per (layer, KV
// head, 32-token block) is scored with the query in the model's own
// attention space.  With pre-RoPE queries on both sides the per-query dot
// products sum to one dot product with the summed query (linearity), so the
// path is: reduce the prefill queries of each KV group to q-bar (one HBM
// pass over q), then stream the index once, a GEMV per unit for all
// sessions at the same time.
#include "common.h"

namespace kvsel {

// q: [S][L][Hq][W][D] -> qbar [S][L][Hkv][D], summed over the group's heads
// and the W tokens.  One workgroup per (s, l, g); 16-byte loads, per-slot
// float64 accumulators, slots reduced in a fixed order, one rounding to
// float32 at the end (the sum of a group's G*W bf16 rows is exact in float64
// unless their magnitudes span more than about 2^30, so q-bar is then the
// correctly rounded sum).
template <int DT>
__global__ __launch_bounds__(256) void query_reduce_kernel(BlockParams p, const void* __restrict__ q,
                                                           float* __restrict__ qbar) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = 16 / esz;
  __shared__ double part[256][8];
  const int unit = blockIdx.x;                  // (s, l, g)
  const int g = unit % p.Hkv;
  const int sl = unit / p.Hkv;                  // s * L + l
  const int G = p.Hq / p.Hkv;
  const int lpr = p.D / E;                      // lanes per row
  const int slots = 256 / lpr;
  const int tid = threadIdx.x;
  const int slot = tid / lpr, rl = tid % lpr;
  const int64_t rows = static_cast<int64_t>(G) * p.W;
  const uint8_t* base = static_cast<const uint8_t*>(q) +
                        ((static_cast<int64_t>(sl) * p.Hq + static_cast<int64_t>(g) * G) * p.W * p.D) * esz;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  // rows slot, slot + slots, ... in order, kRowBatch loads in flight at a time
  constexpr int kRowBatch = 8;
  for (int64_t r0 = slot; r0 < rows; r0 += static_cast<int64_t>(slots) * kRowBatch) {
    uint4 vb[kRowBatch];
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      const int64_t r = r0 + static_cast<int64_t>(j) * slots;
      vb[j] = (r < rows) ? *reinterpret_cast<const uint4*>(base + (r * p.D + rl * E) * esz) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      if (r0 + static_cast<int64_t>(j) * slots >= rows) break;
      const uint32_t w[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
      if constexpr (DT == KVSEL_F32) {
        for (int i = 0; i < 4; ++i) acc[i] += static_cast<double>(__uint_as_float(w[i]));
      } else {
        for (int i = 0; i < 4; ++i) {
          const uint16_t lo = static_cast<uint16_t>(w[i] & 0xFFFFu), hi = static_cast<uint16_t>(w[i] >> 16);
          acc[2 * i] += static_cast<double>((DT == KVSEL_BF16) ? bf16_to_f32(lo) : f16_to_f32(lo));
          acc[2 * i + 1] += static_cast<double>((DT == KVSEL_BF16) ? bf16_to_f32(hi) : f16_to_f32(hi));
        }
      }
    }
  }
  for (int i = 0; i < 8; ++i) part[tid][i] = acc[i];
  __syncthreads();
  for (int d = tid; d < p.D; d += 256) {
    const int l2 = d / E, i = d % E;
    double s = 0.0;
    for (int sl2 = 0; sl2 < slots; ++sl2) s += part[sl2 * lpr + l2][i];
    qbar[static_cast<int64_t>(unit) * p.D + d] = static_cast<float>(s);
  }
}

// out[s][u][b - n_begin] = scale * qbar[s][u] . mu[u][b] for b in the tile.
// 16 bytes of a row per lane (D*2/16 lanes per row), S sessions at once, the
// row dot finished with an xor-shuffle tree across the row's lanes.
template <int S_MAX>
__global__ __launch_bounds__(256) void block_scores_kernel(BlockParams p, const float* __restrict__ qbar,
                                                           const uint16_t* __restrict__ mu,
                                                           float* __restrict__ out) {
  const int U = p.L * p.Hkv;
  const int u = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int lpr = p.D / 8;                      // f16: 8 elements per 16 bytes
  const int rows_per_wave = 64 / lpr;
  const int rl = lane % lpr, rsub = lane / lpr;
  float qb[S_MAX][8];
  for (int s = 0; s < S_MAX; ++s)
    for (int i = 0; i < 8; ++i)
      qb[s][i] = (s < p.S) ? qbar[(static_cast<int64_t>(s) * U + u) * p.D + rl * 8 + i] : 0.f;
  const uint16_t* mu_u = mu + (static_cast<int64_t>(u) * p.NB) * p.D;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * blockDim.x / 64;
  for (int64_t r0 = wave * rows_per_wave; r0 < p.n_count; r0 += n_waves * rows_per_wave) {
    const int64_t r = r0 + rsub;
    const bool ok = r < p.n_count;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ok) v = *reinterpret_cast<const uint4*>(mu_u + (p.n_begin + r) * p.D + rl * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = f16_to_f32(static_cast<uint16_t>(w[i] & 0xFFFFu));
      x[2 * i + 1] = f16_to_f32(static_cast<uint16_t>(w[i] >> 16));
    }
    float acc[S_MAX];
    for (int s = 0; s < S_MAX; ++s) {
      float a = 0.f;
      for (int i = 0; i < 8; ++i) a = fmaf(qb[s][i], x[i], a);
      acc[s] = a;
    }
    for (int o = lpr / 2; o > 0; o >>= 1)
      for (int s = 0; s < S_MAX; ++s) acc[s] += __shfl_xor(acc[s], o, 64);
    if (ok) {
      for (int s = 0; s < S_MAX; ++s)
        if (s < p.S && rl == s) out[(static_cast<int64_t>(s) * U + u) * p.n_count + r] = acc[s] * p.scale;
    }
  }
}

// The same scores on the matrix cores: v_mfma_f32_16x16x16_f16 with 16
// index rows as the A operand and the sessions' q-bar as the B columns.
// q-bar is float32; it enters the f16 products as hi + lo parts after a
// per-session power-of-two scaling (exact), so the products carry about 22
// significant bits.  The contraction over d is split into k-steps in a
// permuted but consistent order on both operands: lane quarter q, k-step
// 2t+h covers d = 8q + 32t + 4h .. +3, so each lane reads 16 contiguous
// bytes of its index row per pair of k-steps.
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each wavefront scores kTilesPerWave consecutive 16-row tiles of one unit
// (a contiguous 64 KiB run of the index), loading the next tile's A
// fragments while the current tile's MFMAs run.  The scores of its 256 rows
// are staged in the wavefront's own LDS rows (one per session, padded to
// avoid bank conflicts) and written at the end as whole 1 KiB runs per
// session: the MFMA layout would otherwise scatter them as 64-byte pieces,
// which costs the HBM write path several times their bytes.
//
// Packed output (a threshold per session and unit given): the wavefront's
// 256 rows are one chunk of the packed tile format; only the scores whose
// key is above the threshold are written, packed at the chunk's start in
// row order, with the chunk's four mask words.  The tiled selection passes
// the threshold from its running set, so after the first tile the stores
// shrink to the few columns that can still enter it: score stores
// interleaved with the index stream cost the read path far more than
// their bytes.
constexpr int kTilesPerWave = 16;
static_assert(kTilesPerWave * 16 == kPackChunk, "one wavefront's rows form one packed chunk");
constexpr int kStageStride = kTilesPerWave * 16 + 4;    // floats per staged session row

__global__ __launch_bounds__(256) void block_scores_mfma_kernel(BlockParams p, const float* __restrict__ qbar,
                                                                const uint16_t* __restrict__ mu,
                                                                float* __restrict__ out) {
  const int U = p.L * p.Hkv;
  const int u = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, quarter = lane >> 4;
  const int64_t n_tiles = (p.n_count + 15) / 16;
  const int64_t t_begin = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kTilesPerWave;
  const int64_t t_end = min(n_tiles, t_begin + kTilesPerWave);
  if (t_begin >= n_tiles) return;                // whole wavefront; the kernel has no barrier
  // B fragments: session `col`, d = 8*quarter + 32t + 4h + j; scaled by 2^-e
  const bool live = col < p.S;
  const float* qb = qbar + (static_cast<int64_t>(col < p.S ? col : 0) * U + u) * 128;
  float qv[4][8];
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qv[t][j] = live ? qb[8 * quarter + 32 * t + j] : 0.f;
      amax = fmaxf(amax, fabsf(qv[t][j]));
    }
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  int e2 = 0;
  frexpf(amax, &e2);                             // amax < 2^e2
  const float down = ldexpf(1.f, 14 - e2), up = ldexpf(p.scale, e2 - 14);
  f16x4 bh[4][2], bl[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = qv[t][4 * h + j] * down;
        const _Float16 hi = static_cast<_Float16>(x);
        bh[t][h][j] = hi;
        bl[t][h][j] = static_cast<_Float16>(x - static_cast<float>(hi));
      }
  const uint16_t* mu_u = mu + (static_cast<int64_t>(u) * p.NB + p.n_begin) * 128;
  // packed output: lane s holds session s's admission key, loaded up front
  uint32_t thr_lane = 0u;
  if (p.admit != nullptr && lane < p.S) thr_lane = admit_key(p.admit[static_cast<int64_t>(lane) * U + u]);
  extern __shared__ float stage_all[];
  float* stage = stage_all + (threadIdx.x >> 6) * p.S * kStageStride;
  auto load = [&](int64_t tile, uint4* a) {
    const int64_t r = tile * 16 + col;           // A row of this lane
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a[t] = (r < p.n_count) ? *reinterpret_cast<const uint4*>(mu_u + r * 128 + 8 * quarter + 32 * t)
                             : make_uint4(0, 0, 0, 0);
  };
  auto score = [&](int64_t tile, const uint4* a) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f16x4 a0 = __builtin_bit_cast(f16x4, make_uint2(a[t].x, a[t].y));
      const f16x4 a1 = __builtin_bit_cast(f16x4, make_uint2(a[t].z, a[t].w));
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, bh[t][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, bl[t][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, bh[t][1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, bl[t][1], acc, 0, 0, 0);
    }
    // lane holds session `col`, index rows tile*16 + 4*quarter + i
    if (live)
      *reinterpret_cast<f32x4*>(stage + col * kStageStride + (tile - t_begin) * 16 + 4 * quarter) =
          f32x4{acc[0] * up, acc[1] * up, acc[2] * up, acc[3] * up};
  };
  uint4 a0[4], a1[4];
  load(t_begin, a0);
  for (int64_t tile = t_begin; tile < t_end; tile += 2) {
    if (tile + 1 < t_end) load(tile + 1, a1);
    score(tile, a0);
    if (tile + 1 < t_end) {
      if (tile + 2 < t_end) load(tile + 2, a0);
      score(tile + 1, a1);
    }
  }
  // the wavefront's own LDS rows: its LDS operations complete in order
  __builtin_amdgcn_wave_barrier();
  const int64_t row0 = t_begin * 16;
  const int rows = static_cast<int>(min(p.n_count, t_end * 16) - row0);
  if (p.admit != nullptr) {
    // chunk row0 / kPackChunk of every session's row: the admitted scores
    // are compacted within the wavefront's LDS row (in row order, behind
    // the read position), then written as one run, and the chunk's four
    // mask words as one 32-byte store (rows past the tile: none admitted)
    const int64_t n_words = (p.n_count + 63) / 64;
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    for (int sess = 0; sess < p.S; ++sess) {
      const int64_t orow = static_cast<int64_t>(sess) * U + u;
      const uint32_t thr = static_cast<uint32_t>(__shfl(static_cast<int>(thr_lane), sess, 64));
      float* srow = stage + sess * kStageStride;
      uint64_t mw[kPackChunk / 64];
      uint32_t before = 0;
#pragma unroll
      for (int j = 0; j < kPackChunk / 64; ++j) {
        const int r = 64 * j + lane;
        const float v = (r < rows) ? srow[r] : 0.f;
        const bool adm = r < rows && score_key(v) > thr;
        const uint64_t m = __ballot(adm);
        // every lane has read its element of this word before any lane
        // writes: the writes land at or below row 64 j + lane
        __builtin_amdgcn_wave_barrier();
        if (adm) srow[before + __popcll(m & lt)] = v;
        mw[j] = m;
        before += static_cast<uint32_t>(__popcll(m));
      }
      __builtin_amdgcn_wave_barrier();
      float* o = out + orow * p.n_count + row0;
      for (uint32_t i = lane; i < before; i += 64) o[i] = srow[i];
      const int n_w = (rows + 63) / 64;
      if (lane < n_w) {
        uint64_t m = mw[0];
#pragma unroll
        for (int j = 1; j < kPackChunk / 64; ++j)
          if (lane == j) m = mw[j];
        p.mask[orow * n_words + row0 / 64 + lane] = m;
      }
    }
    return;
  }
  for (int c = lane; c < p.S * (kTilesPerWave * 4); c += 64) {
    const int sess = c / (kTilesPerWave * 4), j = 4 * (c % (kTilesPerWave * 4));
    if (j >= rows) continue;
    const f32x4 v = *reinterpret_cast<const f32x4*>(stage + sess * kStageStride + j);
    float* o = out + (static_cast<int64_t>(sess) * U + u) * p.n_count + row0 + j;
    if (j + 3 < rows && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(o));
    } else {
      for (int i = 0; i < 4 && j + i < rows; ++i) o[i] = v[i];
    }
  }
}

hipError_t launch_query_reduce(const BlockParams& p, int dt, const void* q, float* qbar,
                               hipStream_t st) {
  const int units = p.S * p.L * p.Hkv;
  if (units == 0) return hipSuccess;
  if (dt == KVSEL_BF16) query_reduce_kernel<KVSEL_BF16><<<units, 256, 0, st>>>(p, q, qbar);
  else if (dt == KVSEL_F16) query_reduce_kernel<KVSEL_F16><<<units, 256, 0, st>>>(p, q, qbar);
  else query_reduce_kernel<KVSEL_F32><<<units, 256, 0, st>>>(p, q, qbar);
  return hipGetLastError();
}

hipError_t launch_block_scores(const BlockParams& p, const float* qbar, const void* mu, float* out,
                               hipStream_t st) {
  const int U = p.L * p.Hkv;
  if (U == 0 || p.n_count == 0 || p.S == 0) return hipSuccess;
  const int rows_per_wave = 64 / (p.D / 8);
  // ~8 rows per wave per block iteration, capped grid; the kernel strides
  const int64_t blocks_x = ceil_div(p.n_count, static_cast<int64_t>(rows_per_wave) * 4 * 8);
  dim3 grid(static_cast<unsigned>(blocks_x < 1 ? 1 : (blocks_x > 4096 ? 4096 : blocks_x)), U);
  const uint16_t* m = static_cast<const uint16_t*>(mu);
  if (p.D == 128) {
    const int64_t bx = ceil_div(ceil_div(p.n_count, 16), 4 * kTilesPerWave);
    if (bx > 2147483647) return hipErrorInvalidValue;
    dim3 g2(static_cast<unsigned>(bx), U);
    const size_t lds = static_cast<size_t>(4) * p.S * kStageStride * sizeof(float);
    block_scores_mfma_kernel<<<g2, 256, lds, st>>>(p, qbar, m, out);
    return hipGetLastError();
  }
  if (p.S <= 1) block_scores_kernel<1><<<grid, 256, 0, st>>>(p, qbar, m, out);
  else if (p.S <= 4) block_scores_kernel<4><<<grid, 256, 0, st>>>(p, qbar, m, out);
  else block_scores_kernel<8><<<grid, 256, 0, st>>>(p, qbar, m, out);
  return hipGetLastError();
}

}  // namespace kvsel
