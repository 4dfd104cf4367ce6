// Incremental update of a paged execution view between consecutive steps.
//
// KVMem (tiered movement): pages that overlap across consecutive steps stay
// on the GPU; missed blocks are scattered in and re-RoPEd at their new
// positions.  Reading taken here (the pages give no placement rule):
//  * a block in both views keeps its page and V; its K is rotated in place by
//    the change of its logical position, (i_new - i_old) * bt;
//  * pages of blocks that left the view are freed and handed, in ascending
//    page order, to the missed blocks in ascending block order;
//  * a missed block gets raw K rotated to pos0 + i_new*bt + o and V copied,
//    both read from the raw source by block id or, when the caller passes
//    packed staging buffers (the missed blocks after their host-to-device
//    copy, in ascending block order), from entry `miss rank` of the staging.
// Hit pages, freed pages and miss pages are disjoint, so all moves run in one
// pass with no conflicts (the concern ActKV §7.2 plans around for in-place
// compaction).
//
// plan kernel: one workgroup per unit.  Membership by binary search over the
// two ascending index lists staged in LDS; freed pages ordered by a bitmap
// over page ids and a prefix count of its words; misses ranked with a
// ballot prefix.  data kernel: one wavefront per (kept entry, K or V): a
// miss's V copy and its K rotation go to different wavefronts, so each holds
// 4 row passes of one stream in flight and the kernel runs 4 wavefronts per
// SIMD (both measured faster than one wavefront moving K and V together).
#include "rope_dev.h"

namespace kvsel {

using namespace rope;

namespace {
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int64_t kMaxPoolPages = 1 << 18;      // bitmap <= 32 KiB
constexpr int kMaxK = 8192;
constexpr int kMaxOffTable = 32 * 64;

__device__ __forceinline__ int find_sorted(const int32_t* a, int n, int32_t x) {
  int lo = 0, hi = n - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int32_t v = a[mid];
    if (v == x) return mid;
    if (v < x) lo = mid + 1;
    else hi = mid - 1;
  }
  return -1;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}
}  // namespace

// The plan per new entry: its previous position i_old (a hit), or -1 - r
// for the miss of rank r among the unit's misses (ascending block order).
size_t incremental_workspace_bytes(const GatherParams& p) {
  return static_cast<size_t>(p.U) * p.k * sizeof(int32_t);
}

__global__ __launch_bounds__(kPlanThreads) void incremental_plan_kernel(
    GatherParams p, const int32_t* __restrict__ idx, const int32_t* __restrict__ prev_idx,
    const int32_t* __restrict__ prev_page, int32_t* __restrict__ page_table,
    int32_t* __restrict__ n_miss, int32_t* __restrict__ plan_old) {
  extern __shared__ uint32_t sm[];
  __shared__ uint32_t wave_cnt[kPlanWaves];
  __shared__ uint32_t word_scan[kPlanThreads];
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k;
  const int64_t nw = (p.pool_pages + 31) / 32;
  int32_t* s_new = reinterpret_cast<int32_t*>(sm);
  int32_t* s_prev = s_new + k;
  int32_t* s_freed = s_prev + k;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(s_freed + k);
  const int32_t* new_u = idx + static_cast<int64_t>(u) * k;
  const int32_t* prev_u = prev_idx + static_cast<int64_t>(u) * k;
  const int32_t* ppage_u = prev_page + static_cast<int64_t>(u) * k;
  for (int i = tid; i < k; i += kPlanThreads) {
    s_new[i] = new_u[i];
    s_prev[i] = prev_u[i];
    s_freed[i] = -1;
  }
  for (int64_t w = tid; w < nw; w += kPlanThreads) bitmap[w] = 0u;
  __syncthreads();
  // pages of previous blocks that are not in the new view
  for (int i = tid; i < k; i += kPlanThreads) {
    if (find_sorted(s_new, k, s_prev[i]) < 0) {
      const int32_t pg = ppage_u[i];
      if (pg >= 0 && pg < p.pool_pages) atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
    }
  }
  __syncthreads();
  // rank of each freed page = number of freed pages with a smaller id
  const int64_t wpt = (nw + kPlanThreads - 1) / kPlanThreads;
  const int64_t w0 = min(nw, static_cast<int64_t>(tid) * wpt), w1 = min(nw, w0 + wpt);
  uint32_t cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
  word_scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {       // inclusive scan
    const uint32_t v = (tid >= off) ? word_scan[tid - off] : 0u;
    __syncthreads();
    word_scan[tid] += v;
    __syncthreads();
  }
  uint32_t rank = word_scan[tid] - cnt;
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      if (rank < static_cast<uint32_t>(k)) s_freed[rank] = static_cast<int32_t>(w * 32 + b);
      ++rank;
    }
  }
  __syncthreads();
  // misses in ascending order take the freed pages in ascending order
  const int seg = ((k + kPlanWaves - 1) / kPlanWaves + 63) / 64 * 64;
  const int s_beg = min(k, wave * seg), s_end = min(k, s_beg + seg);
  uint32_t nm = 0;
  for (int i0 = s_beg; i0 < s_end; i0 += 64) {
    const int i = i0 + lane;
    const bool miss = i < s_end && find_sorted(s_prev, k, s_new[i]) < 0;
    nm += __popcll(__ballot(miss));
  }
  if (lane == 0) wave_cnt[wave] = nm;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wave_cnt[w];
  int32_t* pt_u = page_table + static_cast<int64_t>(u) * k;
  int32_t* old_u = plan_old + static_cast<int64_t>(u) * k;
  for (int i0 = s_beg; i0 < s_end; i0 += 64) {
    const int i = i0 + lane;
    int io = -1;
    if (i < s_end) io = find_sorted(s_prev, k, s_new[i]);
    const bool miss = i < s_end && io < 0;
    const uint64_t b = __ballot(miss);
    if (i < s_end) {
      if (miss) {
        const uint32_t r = base + __popcll(b & lanemask_lt(lane));
        pt_u[i] = (r < static_cast<uint32_t>(k)) ? s_freed[r] : -1;
        old_u[i] = -1 - static_cast<int32_t>(r);
      } else {
        pt_u[i] = ppage_u[io];
        old_u[i] = io;
      }
    }
    base += __popcll(b);
  }
  if (tid == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kPlanWaves; ++w) t += wave_cnt[w];
    n_miss[u] = static_cast<int32_t>(t);
  }
}

template <int DT, bool kInter, bool kRot>
__global__ __launch_bounds__(256) void incremental_data_kernel(
    GatherParams p, RopeTable rt, const void* __restrict__ src_k, const void* __restrict__ src_v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ plan_old, void* __restrict__ pool_k, void* __restrict__ pool_v) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = Vec16<DT>::kElems;
  constexpr int NP = kInter ? E / 2 : E;     // pairs touched by this lane
  constexpr int kBatch = 4;                  // row passes whose loads are in flight together
  __shared__ float2 off_tab[kMaxOffTable];
  const int half = p.D / 2;
  if constexpr (kRot) {
    for (int t = threadIdx.x; t < p.bt * half; t += blockDim.x) {
      const int o = t / half, m = t - (t / half) * half;
      float c, s;
      angle_sincos(static_cast<double>(o), rt.inv_freq[m], &c, &s);
      off_tab[t] = make_float2(c, s);
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int lpr = p.D * esz / 16;
  const int rows_per_pass = 64 / lpr;
  const int rlane = lane % lpr, rsub = lane / lpr;
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

  // work item tt: entry tt / 2, its K (even) or V (odd).  The next item's
  // plan entries are loaded while the current item moves.
  int32_t page_n = 0, io_n = 0, blk_n = 0;
  if (wave_global < 2 * items) {
    page_n = page_table[wave_global >> 1];
    io_n = plan_old[wave_global >> 1];
    blk_n = idx[wave_global >> 1];
  }
  for (int64_t tt = wave_global; tt < 2 * items; tt += n_waves) {
    const int64_t it = tt >> 1;
    const bool vhalf = (tt & 1) != 0;
    const int u = static_cast<int>(it / p.k);
    const int64_t i = it - static_cast<int64_t>(u) * p.k;
    const int32_t page = page_n, io = io_n, blk = blk_n;
    if (tt + n_waves < 2 * items) {
      page_n = page_table[(tt + n_waves) >> 1];
      io_n = plan_old[(tt + n_waves) >> 1];
      blk_n = idx[(tt + n_waves) >> 1];
    }
    if (page < 0 || page >= p.pool_pages) continue;
    uint8_t* pk = static_cast<uint8_t*>(pool_k) + (static_cast<int64_t>(u) * p.pool_pages + page) * item_bytes;
    uint8_t* pv = static_cast<uint8_t*>(pool_v) + (static_cast<int64_t>(u) * p.pool_pages + page) * item_bytes;
    const bool hit = io >= 0;
    // a hit whose position moved gets its K anew (V untouched): rotated in
    // place by (i - io) * bt, or, with hit_raw, its raw K from the source
    // rotated to the new position; a miss is raw K rotated to its new
    // position, with V copied
    if (hit && (i == io || !kRot)) continue;
    const bool from_src = !hit || p.hit_raw;
    const int64_t angle_pos = from_src ? p.pos0 + i * p.bt : (i - io) * p.bt;
    const uint8_t* sk = nullptr;
    const uint8_t* sv = nullptr;
    if (hit && p.hit_raw) {
      const int32_t b = blk;
      if (b < 0 || (static_cast<int64_t>(b) + 1) * p.bt > p.src_rows) continue;
      const int64_t soff = p.src_offsets ? p.src_offsets[u] : static_cast<int64_t>(u) * p.src_unit_stride;
      sk = static_cast<const uint8_t*>(p.hit_src) + soff * esz + static_cast<int64_t>(b) * item_bytes;
    } else if (!hit && p.staged_cap >= 0) {
      // packed staging: the miss of rank r is entry r of the unit's buffers
      const int64_t r = -1 - static_cast<int64_t>(io);
      if (r >= p.staged_cap) continue;
      const int64_t e = static_cast<int64_t>(u) * p.staged_cap + r;
      sk = static_cast<const uint8_t*>(src_k) + e * item_bytes;
      sv = static_cast<const uint8_t*>(src_v) + e * item_bytes;
    } else if (!hit) {
      const int32_t b = blk;
      if (b < 0 || (static_cast<int64_t>(b) + 1) * p.bt > p.src_rows) continue;
      const int64_t soff = p.src_offsets ? p.src_offsets[u] : static_cast<int64_t>(u) * p.src_unit_stride;
      sk = static_cast<const uint8_t*>(src_k) + soff * esz + static_cast<int64_t>(b) * item_bytes;
      sv = static_cast<const uint8_t*>(src_v) + soff * esz + static_cast<int64_t>(b) * item_bytes;
    }
    if (vhalf) {
      // V: copied for a miss, untouched for a hit
      if (hit) continue;
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
            store16_stream(pv + static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz, vv[j]);
        }
      }
      continue;
    }
    float cb[NP], sb[NP];
    if constexpr (kRot) {
      float cl = 1.f, sl = 0.f;
      if (lane < half) angle_sincos(static_cast<double>(angle_pos), rt.inv_freq[lane], &cl, &sl);
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        cb[e] = __shfl(cl, m0 + e, 64);
        sb[e] = __shfl(sl, m0 + e, 64);
      }
    }
    for (int q0 = 0; q0 < passes; q0 += kBatch) {
      uint4 kv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int o = (q0 + j) * rows_per_pass + rsub;
        kv[j] = make_uint4(0, 0, 0, 0);
        if (q0 + j < passes && o < p.bt) {
          const int64_t off = static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz;
          kv[j] = *reinterpret_cast<const uint4*>((from_src ? sk : pk) + off);
        }
      }

#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (q0 + j >= passes) break;                    // uniform
        const int o = (q0 + j) * rows_per_pass + rsub;
        uint4 out = kv[j];
        if constexpr (kRot) {
          const uint4 other = kInter ? kv[j] : shfl16(kv[j], partner);
          float cs[NP], sn[NP];
          if (!from_src) {
#pragma unroll
            for (int e = 0; e < NP; ++e) {
              cs[e] = cb[e];
              sn[e] = sb[e];
            }
          } else {
            const float4* t4 = reinterpret_cast<const float4*>(&off_tab[(o < p.bt ? o : 0) * half + m0]);
#pragma unroll
            for (int e = 0; e < NP; e += 2) {
              const float4 t = t4[e / 2];
              add_angles(cb[e], sb[e], t.x, t.y, &cs[e], &sn[e]);
              add_angles(cb[e + 1], sb[e + 1], t.z, t.w, &cs[e + 1], &sn[e + 1]);
            }
          }
          out = rotate16<DT, kInter>(kv[j], other, sgn, cs, sn);
        }
        if (o < p.bt) {
          const int64_t off = static_cast<int64_t>(o) * row_bytes + static_cast<int64_t>(d0) * esz;
          store16_stream(pk + off, out);
        }
      }
    }
  }
}

hipError_t launch_gather_incremental(const GatherParams& p, const RopeTable& rt, const void* src_k,
                                     const void* src_v, const int32_t* idx, const int32_t* prev_idx,
                                     const int32_t* prev_page, void* pool_k, void* pool_v,
                                     int32_t* page_table, int32_t* n_miss, void* ws, hipStream_t st) {
  if (p.U == 0 || p.k == 0) return hipSuccess;
  if (p.k > kMaxK || p.pool_pages > kMaxPoolPages || p.rotary_dim != p.D ||
      (p.rope == KVSEL_ROPE_RAW && p.bt * (p.D / 2) > kMaxOffTable))
    return hipErrorNotSupported;
  int32_t* plan_old = static_cast<int32_t*>(ws);
  const size_t sh = static_cast<size_t>(p.k) * 3 * 4 + static_cast<size_t>((p.pool_pages + 31) / 32) * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&incremental_plan_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sh));
  if (e != hipSuccess) return e;
  incremental_plan_kernel<<<p.U, kPlanThreads, sh, st>>>(p, idx, prev_idx, prev_page, page_table, n_miss,
                                                         plan_old);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t items = static_cast<int64_t>(p.U) * p.k;
  const int64_t blocks = ceil_div(items, 4);
  const int grid = static_cast<int>(blocks > 65536 ? 65536 : blocks);
#define KVSEL_ID3(DTV, INTER, ROT)                                                                 \
  incremental_data_kernel<DTV, INTER, ROT><<<grid, 256, 0, st>>>(p, rt, src_k, src_v, idx, page_table,  \
                                                                 plan_old, pool_k, pool_v)
#define KVSEL_ID(DTV)                                                                              \
  do {                                                                                             \
    const bool inter = p.style == KVSEL_ROPE_INTERLEAVED, rot = p.rope == KVSEL_ROPE_RAW;          \
    if (inter) {                                                                                   \
      if (rot) KVSEL_ID3(DTV, true, true); else KVSEL_ID3(DTV, true, false);                       \
    } else {                                                                                       \
      if (rot) KVSEL_ID3(DTV, false, true); else KVSEL_ID3(DTV, false, false);                     \
    }                                                                                              \
  } while (0)
  if (p.dtype == KVSEL_BF16) KVSEL_ID(KVSEL_BF16);
  else if (p.dtype == KVSEL_F16) KVSEL_ID(KVSEL_F16);
  else KVSEL_ID(KVSEL_F32);
#undef KVSEL_ID
#undef KVSEL_ID3
  return hipGetLastError();
}

}  // namespace kvsel
