// Gather of kept entries into a compact view, with optional re-RoPE of K.
//
// KVMem (tiered movement): selected blocks are packed into contiguous
// logical positions; raw, position-free K is rotated for its new position
// and V is copied unchanged.
//
// Two kernels:
//  * rows: one row (D elements) per group of D*esz/16 lanes, 16 bytes per
//    lane.  Any bt; RoPE angles computed per lane.  Used for token gathers.
//  * blocks: one wavefront per (kept entry, K or V) of bt >= 8 rows with
//    RoPE: the V copy and the K rotation of an entry go to different
//    wavefronts (measured 11 % faster than one wavefront moving both; for
//    single rows the split measured slower, so the rows kernel keeps both).
//    The rotation of row o at base position b is composed from a per-entry
//    base rotation (one sincos per frequency and lane) and a per-workgroup
//    table of the offsets o (angle addition), so trigonometry is amortised
//    over bt rows.  Angles are formed and range-reduced in float64.
#include "rope_dev.h"

namespace kvsel {

using namespace rope;

namespace {

__device__ __forceinline__ const uint8_t* unit_src(const void* base, const GatherParams& p, int u,
                                                   int esz) {
  const int64_t off = p.src_offsets ? p.src_offsets[u] : static_cast<int64_t>(u) * p.src_unit_stride;
  return static_cast<const uint8_t*>(base) + off * esz;
}

}  // namespace

// ------------------------------------------------------------------ rows kernel
template <int DT>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherParams p, RopeTable rt,
                                                          const void* __restrict__ src_k,
                                                          const void* __restrict__ src_v,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ n_idx,
                                                          void* __restrict__ dst_k,
                                                          void* __restrict__ dst_v) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = Vec16<DT>::kElems;
  const int lpr = p.D * esz / 16;          // lanes per row
  const int rows_per_wave = 64 / lpr;
  const int lane = threadIdx.x & 63;
  const int rlane = lane % lpr;            // lane within its row
  const int rsub = lane / lpr;             // row slot within the wave
  const int64_t rows_per_unit = static_cast<int64_t>(p.k) * p.bt;
  const int64_t total_rows = rows_per_unit * p.U;
  const int64_t wave_global = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * blockDim.x / 64;
  const int rd = p.rotary_dim;
  const int d0 = rlane * E;
  const bool interleaved = p.style == KVSEL_ROPE_INTERLEAVED;
  const int half_lanes = (rd / 2) / E;
  const bool in_rot = d0 < rd;
  const bool first = d0 < rd / 2;
  const int partner = first ? lane + half_lanes : lane - half_lanes;

  for (int64_t r0 = wave_global * rows_per_wave; r0 < total_rows; r0 += n_waves * rows_per_wave) {
    const int64_t r = r0 + rsub;
    bool active = r < total_rows && rsub < rows_per_wave;
    int u = 0;
    int64_t i = 0, o = 0, srow = 0;
    if (active) {
      u = static_cast<int>(r / rows_per_unit);
      const int64_t rr = r - static_cast<int64_t>(u) * rows_per_unit;
      i = rr / p.bt;
      o = rr - i * p.bt;
      const int32_t b = idx[static_cast<int64_t>(u) * p.k + i];
      const bool valid_i = n_idx == nullptr || i < n_idx[u];
      srow = static_cast<int64_t>(b) * p.bt + o;
      active = valid_i && b >= 0 && srow < p.src_rows;
    }
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (active) {
      const int64_t off = (srow * p.D) * esz + static_cast<int64_t>(d0) * esz;
      kv = *reinterpret_cast<const uint4*>(unit_src(src_k, p, u, esz) + off);
      vv = *reinterpret_cast<const uint4*>(unit_src(src_v, p, u, esz) + off);
    }
    if (p.rope != KVSEL_ROPE_NONE) {
      const uint4 other = interleaved ? kv : shfl16(kv, partner);
      if (active && in_rot) {
        const int64_t pnew = p.pos0 + i * p.bt + o;
        const double pos = (p.rope == KVSEL_ROPE_RAW) ? static_cast<double>(pnew)
                                                      : static_cast<double>(pnew - srow);
        float cs[E], sn[E];
        const int npair = interleaved ? E / 2 : E;
        for (int e = 0; e < npair; ++e) {
          const int m = interleaved ? (d0 / 2 + e) : ((d0 % (rd / 2)) + e);
          angle_sincos(pos, rt.inv_freq[m], &cs[e], &sn[e]);
        }
        kv = rotate_chunk<DT>(kv, other, first, interleaved, cs, sn);
      }
    }
    if (active) {
      const int64_t doff = ((static_cast<int64_t>(u) * rows_per_unit + i * p.bt + o) * p.D) * esz +
                           static_cast<int64_t>(d0) * esz;
      store16_stream(static_cast<uint8_t*>(dst_k) + doff, kv);
      store16_stream(static_cast<uint8_t*>(dst_v) + doff, vv);
    }
  }
}

// ------------------------------------------------------------------ blocks kernel
// Requires rotary_dim == D, bt * (D/2) <= kMaxOffTable, bt rows per entry.
constexpr int kMaxOffTable = 32 * 64;

template <int DT, bool kInter, bool kRaw>
__global__ __launch_bounds__(256) void gather_blocks_kernel(GatherParams p, RopeTable rt,
                                                            const void* __restrict__ src_k,
                                                            const void* __restrict__ src_v,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ n_idx,
                                                            void* __restrict__ dst_k,
                                                            void* __restrict__ dst_v) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = Vec16<DT>::kElems;
  constexpr int NP = kInter ? E / 2 : E;     // pairs touched by this lane
  constexpr int kBatch = 8;                 // row passes whose loads are in flight together
  __shared__ float2 off_tab[kMaxOffTable];   // (cos, sin) of o * inv_freq[m], [o][m]
  const int half = p.D / 2;
  if constexpr (kRaw) {
    for (int t = threadIdx.x; t < p.bt * half; t += blockDim.x) {
      const int o = t / half, m = t - (t / half) * half;
      float c, s;
      angle_sincos(static_cast<double>(o), rt.inv_freq[m], &c, &s);
      off_tab[t] = make_float2(c, s);
    }
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int lpr = p.D * esz / 16;               // lanes per row
  const int rows_per_pass = 64 / lpr;
  const int rlane = lane % lpr;
  const int rsub = lane / lpr;
  const int d0 = rlane * E;
  const bool first = d0 < half;
  const float sgn = first ? -1.f : 1.f;
  const int partner = first ? lane + lpr / 2 : lane - lpr / 2;
  const int m0 = kInter ? d0 / 2 : (d0 % half);
  const int64_t items = static_cast<int64_t>(p.U) * p.k;
  const int64_t wave_global = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * blockDim.x / 64;
  const int64_t row_bytes = static_cast<int64_t>(p.D) * esz;
  const int64_t item_bytes = row_bytes * p.bt;
  const int passes = (p.bt + rows_per_pass - 1) / rows_per_pass;

  // work item tt: entry tt / 2, its K (even) or V (odd).  With an even
  // n_waves a wavefront takes the other half of its entry on odd passes
  // (tt0 ^ 1: the same entry, each item still taken once), so every
  // wavefront alternates between K items (rotated) and V items (copied).
  int32_t b_n = (wave_global < 2 * items) ? idx[wave_global >> 1] : 0;
  int64_t pass = 0;
  for (int64_t tt0 = wave_global; tt0 < 2 * items; tt0 += n_waves, ++pass) {
    const int64_t tt = (n_waves & 1) ? tt0 : (tt0 ^ (pass & 1));
    const int64_t it = tt >> 1;
    const int u = static_cast<int>(it / p.k);
    const int64_t i = it - static_cast<int64_t>(u) * p.k;
    const int32_t b = b_n;
    if (tt0 + n_waves < 2 * items) b_n = idx[(tt0 + n_waves) >> 1];
    if (n_idx != nullptr && i >= n_idx[u]) continue;
    if (b < 0 || (static_cast<int64_t>(b) + 1) * p.bt > p.src_rows) continue;
    if (tt & 1) {
      const uint8_t* sv = unit_src(src_v, p, u, esz) + static_cast<int64_t>(b) * item_bytes;
      uint8_t* dv = static_cast<uint8_t*>(dst_v) + it * item_bytes;
      for (int q0 = 0; q0 < passes; q0 += kBatch) {
        uint4 vv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int o = (q0 + j) * rows_per_pass + rsub;
          vv[j] = make_uint4(0, 0, 0, 0);
          if (q0 + j < passes && o < p.bt)
            vv[j] = *reinterpret_cast<const uint4*>(sv + static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int o = (q0 + j) * rows_per_pass + rsub;
          if (q0 + j < passes && o < p.bt)
            store16_stream(dv + static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz, vv[j]);
        }
      }
      continue;
    }
    const uint8_t* sk = unit_src(src_k, p, u, esz) + static_cast<int64_t>(b) * item_bytes;
    uint8_t* dk = static_cast<uint8_t*>(dst_k) + it * item_bytes;
    // rotation of the item's base position: lane m evaluates frequency m once,
    // the lanes that need it read it across the wavefront
    const int64_t base_pos = kRaw ? p.pos0 + i * p.bt : p.pos0 + (i - b) * p.bt;
    float cl = 1.f, sl = 0.f;
    if (lane < half) angle_sincos(static_cast<double>(base_pos), rt.inv_freq[lane], &cl, &sl);
    float cb[NP], sb[NP];
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      cb[e] = __shfl(cl, m0 + e, 64);
      sb[e] = __shfl(sl, m0 + e, 64);
    }
    for (int q0 = 0; q0 < passes; q0 += kBatch) {
      uint4 kv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int o = (q0 + j) * rows_per_pass + rsub;
        kv[j] = make_uint4(0, 0, 0, 0);
        if (q0 + j < passes && o < p.bt)
          kv[j] = *reinterpret_cast<const uint4*>(sk + static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (q0 + j >= passes) break;                    // uniform
        const int o = (q0 + j) * rows_per_pass + rsub;
        const uint4 other = kInter ? kv[j] : shfl16(kv[j], partner);
        if (o < p.bt) {
          float cs[NP], sn[NP];
          if constexpr (kRaw) {
            const float4* t4 = reinterpret_cast<const float4*>(&off_tab[o * half + m0]);
#pragma unroll
            for (int e = 0; e < NP; e += 2) {
              const float4 t = t4[e / 2];
              add_angles(cb[e], sb[e], t.x, t.y, &cs[e], &sn[e]);
              add_angles(cb[e + 1], sb[e + 1], t.z, t.w, &cs[e + 1], &sn[e + 1]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < NP; ++e) {
              cs[e] = cb[e];
              sn[e] = sb[e];
            }
          }
          const int64_t off = static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz;
          store16_stream(dk + off, rotate16<DT, kInter>(kv[j], other, sgn, cs, sn));
        }
      }
    }
  }
}

static int grid_for(int64_t waves_wanted) {
  const int64_t blocks = ceil_div(waves_wanted, 4);
  return static_cast<int>(blocks < 1 ? 1 : (blocks > 65536 ? 65536 : blocks));
}

hipError_t launch_gather_fresh(const GatherParams& p, const RopeTable& rt, const void* src_k,
                               const void* src_v, const int32_t* idx, const int32_t* n_idx,
                               void* dst_k, void* dst_v, hipStream_t st) {
  if (p.U == 0 || p.k == 0) return hipSuccess;
  const int esz = p.dtype == KVSEL_F32 ? 4 : 2;
  const int lpr = p.D * esz / 16;
  const bool blocks_path = p.rope != KVSEL_ROPE_NONE && p.bt >= 8 && p.rotary_dim == p.D &&
                           p.bt * (p.D / 2) <= kMaxOffTable && lpr <= 64;
  if (blocks_path) {
    const int grid = grid_for(static_cast<int64_t>(p.U) * p.k);
#define KVSEL_GB3(DTV, INTER, RAW)                                                              \
  gather_blocks_kernel<DTV, INTER, RAW><<<grid, 256, 0, st>>>(p, rt, src_k, src_v, idx, n_idx, dst_k, dst_v)
#define KVSEL_GB(DTV)                                                                           \
  do {                                                                                          \
    const bool inter = p.style == KVSEL_ROPE_INTERLEAVED, raw = p.rope == KVSEL_ROPE_RAW;       \
    if (inter) {                                                                                \
      if (raw) KVSEL_GB3(DTV, true, true); else KVSEL_GB3(DTV, true, false);                    \
    } else {                                                                                    \
      if (raw) KVSEL_GB3(DTV, false, true); else KVSEL_GB3(DTV, false, false);                  \
    }                                                                                           \
  } while (0)
    if (p.dtype == KVSEL_BF16) KVSEL_GB(KVSEL_BF16);
    else if (p.dtype == KVSEL_F16) KVSEL_GB(KVSEL_F16);
    else KVSEL_GB(KVSEL_F32);
#undef KVSEL_GB
#undef KVSEL_GB3
  } else {
    const int64_t rows = static_cast<int64_t>(p.U) * p.k * p.bt;
    const int rows_per_wave = 64 / lpr;
    // one pass of rows per wavefront where the grid cap allows (more
    // wavefronts in flight measured faster than longer strides per wavefront)
    const int grid = grid_for(ceil_div(rows, static_cast<int64_t>(rows_per_wave)));
#define KVSEL_GR(DTV)                                                                         \
  gather_rows_kernel<DTV><<<grid, 256, 0, st>>>(p, rt, src_k, src_v, idx, n_idx, dst_k, dst_v)
    if (p.dtype == KVSEL_BF16) KVSEL_GR(KVSEL_BF16);
    else if (p.dtype == KVSEL_F16) KVSEL_GR(KVSEL_F16);
    else KVSEL_GR(KVSEL_F32);
#undef KVSEL_GR
  }
  return hipGetLastError();
}

}  // namespace kvsel
