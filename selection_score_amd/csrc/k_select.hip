// Budgeted top-k with a forced set, restored to chronological order.
//
// IntentKV §4 (top-k selection): keep the forced set plus the best of the
// rest up to the budget.  KVMem (query-conditioned retrieval): sink and
// recent entries are forced, the rest is filled by score, and the result is
// listed in chronological order.  IntentKV §3: dead positions are never
// candidates.
//
// One workgroup (16 wavefronts) per unit.  Scores become order-preserving
// uint32 keys; an MSB-first 8-bit radix select over LDS histograms finds the
// threshold key T and how many entries equal to T to take.  Ties at T go to
// the lower index: the candidate sequence (running candidates from earlier
// tiles, then this tile's columns) is in ascending global index, and a
// ballot-based prefix count over it ranks the T-valued entries.  A second
// ballot prefix places the selected entries, which therefore come out in
// ascending index order without a sort.
//
// Most calls run in two launches.  select_keys_kernel spreads the unit over
// many workgroups: it stages a 4096-column slice of the score row (plus the
// pooling halo) in LDS, writes the pooled key of every column to the
// workspace and a 256-bin histogram of the keys' top byte per slice.  The
// per-unit workgroup then sums those histograms (the first radix pass) and
// runs the remaining passes and both sweeps: with up to 32 keys per thread
// held in registers (select_regs_kernel, untiled calls), otherwise reading
// the workspace (select_kernel; tiled calls stage their running candidates
// in LDS ahead of the tile's keys).  Untiled calls without a slot map --
// unpooled, max-pooled with a window of up to 9, or average-pooled with a
// window of up to 9 over rows of at most 2048 -- with at least 128 units of
// up to 32768 columns or with rows of at most 8192 skip the first launch:
// each unit's workgroup reads its scores, pools them in registers and makes
// its keys itself.  At most 8 units of rows longer than 32768 spread the
// later radix steps over the slices as well (slice_*_kernel).
#include "common.h"

namespace kvsel {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int64_t kLdsKeysMax = 32768;   // tile keys kept in LDS up to this many

struct SelShared {
  uint32_t hist[256];
  uint32_t wave_eq[kWaves];
  uint32_t wave_gt[kWaves];
  uint32_t wave_cnt[kWaves];
  uint32_t wave_sums[3 * kWaves];
  uint32_t prefix;
  int32_t remaining;
  int32_t forced_sink_alive;
  int32_t forced_recent_alive;
};

struct Ctx {
  const float* row;
  int pool, pool_r;      // on-the-fly pooling of the row (untiled calls)
  const uint32_t* ckey;  // running candidates (LDS)
  const int32_t* cidx;
  const uint32_t* tkey;  // tile keys (LDS) or nullptr
  int c0;
  int64_t n, base, sink_end, rec_begin;
  const int32_t* slot_map;
  int64_t dead;
};

__device__ __forceinline__ bool alive_at(const Ctx& c, int64_t g) {
  return c.slot_map == nullptr || static_cast<int64_t>(c.slot_map[g]) != c.dead;
}

__device__ __forceinline__ bool forced_at(const Ctx& c, int64_t g) {
  return g < c.sink_end || g >= c.rec_begin;
}

// Score of tile column j, pooled over the in-range window if asked.
__device__ __forceinline__ float column_score(const Ctx& c, int64_t j) {
  if (c.pool == KVSEL_POOL_NONE) return c.row[j];
  const int64_t lo = max(static_cast<int64_t>(0), j - c.pool_r);
  const int64_t hi = min(c.n - 1, j + c.pool_r);
  if (c.pool == KVSEL_POOL_MAX) {
    float m = c.row[lo];
    for (int64_t i = lo + 1; i <= hi; ++i) m = fmaxf(m, c.row[i]);
    return m;
  }
  float s = 0.f;
  for (int64_t i = j - c.pool_r; i <= j + c.pool_r; ++i) s += (i >= lo && i <= hi) ? c.row[i] : 0.f;
  return s / static_cast<float>(2 * c.pool_r + 1);
}

// Key of virtual entry e (0 = not a candidate) and its global index.
__device__ __forceinline__ uint32_t entry_key(const Ctx& c, int64_t e, int64_t* gidx) {
  if (e < c.c0) {
    *gidx = c.cidx[e];
    return c.ckey[e];
  }
  const int64_t j = e - c.c0;
  const int64_t g = c.base + j;
  *gidx = g;
  if (c.tkey != nullptr) return c.tkey[j];
  if (forced_at(c, g) || !alive_at(c, g)) return 0u;
  return score_key(column_score(c, j));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

// Block-wide sum of a per-thread value (all threads must call).
__device__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < kWaves; ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// Block-wide sums of three per-thread values with one exchange (all threads
// must call).  scratch holds 3 * kWaves words.
__device__ uint3 block_sum3(uint32_t a, uint32_t b, uint32_t c, uint32_t* scratch, int nw = kWaves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
    c += __shfl_xor(c, o, 64);
  }
  __syncthreads();
  if (lane == 0) {
    scratch[wave] = a;
    scratch[nw + wave] = b;
    scratch[2 * nw + wave] = c;
  }
  __syncthreads();
  uint3 t = make_uint3(0u, 0u, 0u);
  for (int w = 0; w < nw; ++w) {
    t.x += scratch[w];
    t.y += scratch[nw + w];
    t.z += scratch[2 * nw + w];
  }
  return t;
}

constexpr int kPrepKeys = 4096;       // columns per select_keys_kernel workgroup
constexpr int kFusedMinUnits = 128;   // untiled calls with this many units make their own keys
constexpr int kFusedSmallN = 8192;    // ... as do calls of any unit count over rows this short
constexpr int kFusedMaxPoolR = 4;     // ... with pooling up to pool_k 9 done in registers (average
constexpr int kFusedAvgKpt = 8;       //     windows only on rows of at most 8 keys per thread)
constexpr int kPrepThreads = 256;
constexpr int kMaxPoolR = 127;        // pool_k <= 255

// Wave 0 of the workgroup: the bin of digit `shift` that holds the
// sh.remaining-th largest candidate among keys matching `prefix` above it
// (sh.hist holds the digit's histogram); updates sh.prefix and sh.remaining.
__device__ __forceinline__ void find_bin(SelShared& sh, uint32_t prefix, int shift, int lane) {
  // lane l owns bins 4l..4l+3
  uint32_t h[4];
  uint32_t own = 0;
  for (int i = 0; i < 4; ++i) {
    h[i] = sh.hist[4 * lane + i];
    own += h[i];
  }
  // inclusive suffix sum over lanes (lanes above me plus mine)
  uint32_t suf = own;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  const uint32_t above_lane = suf - own;   // bins above my range
  const int32_t rem = sh.remaining;
  uint32_t acc = above_lane;
  int found = -1;
  uint32_t above_bin = 0;
  if (above_lane < static_cast<uint32_t>(rem) && suf >= static_cast<uint32_t>(rem)) {
    for (int i = 3; i >= 0; --i) {
      if (acc + h[i] >= static_cast<uint32_t>(rem)) {
        found = 4 * lane + i;
        above_bin = acc;
        break;
      }
      acc += h[i];
    }
  }
  if (found >= 0) {
    sh.prefix = prefix | (static_cast<uint32_t>(found) << shift);
    sh.remaining = rem - static_cast<int32_t>(above_bin);
  }
}

}  // namespace

// Keys of one 4096-column slice of a unit (0 = not a candidate: forced,
// dead, or outside the row) and the histogram of their top byte.
__global__ __launch_bounds__(kPrepThreads) void select_keys_kernel(SelectParams p, const float* scores,
                                                                    uint32_t* keys, uint32_t* hist) {
  __shared__ float row_s[kPrepKeys + 2 * kMaxPoolR];
  __shared__ uint32_t h[256];
  const int u = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kPrepKeys;
  const int jn = static_cast<int>(min(static_cast<int64_t>(kPrepKeys), p.n - j0));
  const int r = (p.pool == KVSEL_POOL_NONE) ? 0 : p.pool_k / 2;
  const float* row = scores + static_cast<int64_t>(u) * p.row_stride;
  const int64_t sink_end = min(static_cast<int64_t>(p.n_sink), p.n_total);
  const int64_t rec_begin = max(sink_end, p.n_total - static_cast<int64_t>(p.n_recent));
  for (int b = tid; b < 256; b += kPrepThreads) h[b] = 0u;
  // row[j0 - r, j0 + jn + r), out-of-range columns as 0 (the AVG convention)
  for (int i = tid; i < jn + 2 * r; i += kPrepThreads) {
    const int64_t j = j0 - r + i;
    row_s[i] = (j >= 0 && j < p.n) ? row[j] : 0.f;
  }
  __syncthreads();
  uint32_t* kout = keys + static_cast<int64_t>(u) * p.n + j0;
  for (int i = tid; i < jn; i += kPrepThreads) {
    const int64_t j = j0 + i;                       // column of the tile
    const int64_t gj = p.base + j;                  // global position
    uint32_t key = 0u;
    const bool alive = p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[gj]) != p.dead_slot;
    if (gj >= sink_end && gj < rec_begin && alive) {
      float v;
      if (p.pool == KVSEL_POOL_MAX) {
        const int lo = static_cast<int>(max(static_cast<int64_t>(0), j - r) - (j0 - r));
        const int hi = static_cast<int>(min(p.n - 1, j + r) - (j0 - r));
        v = row_s[lo];
        for (int t = lo + 1; t <= hi; ++t) v = fmaxf(v, row_s[t]);
      } else if (p.pool == KVSEL_POOL_AVG) {
        v = 0.f;
        for (int t = i; t <= i + 2 * r; ++t) v += row_s[t];
        v = v / static_cast<float>(2 * r + 1);
      } else {
        v = row_s[i];
      }
      key = score_key(v);
      atomicAdd(&h[key >> 24], 1u);
    }
    kout[i] = key;
  }
  __syncthreads();
  uint32_t* hout = hist + (static_cast<int64_t>(u) * gridDim.x + blockIdx.x) * 256;
  for (int b = tid; b < 256; b += kPrepThreads) hout[b] = h[b];
}

// Per-unit selection.  MODE: kPrepared (keys and top-byte histograms from
// select_keys_kernel), kLdsKeys (tiled, tile keys staged in LDS), kOnTheFly
// (tiled, keys recomputed from the scores at every sweep).
enum SelectMode { kPrepared = 0, kLdsKeys = 1, kOnTheFly = 2 };

template <int MODE>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectParams p, const float* scores,
                                                          const uint32_t* prep_keys,
                                                          const uint32_t* prep_hist, int n_slices) {
  extern __shared__ uint32_t dyn[];
  __shared__ SelShared sh;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  Ctx c;
  c.row = scores + static_cast<int64_t>(u) * p.row_stride;
  c.pool = p.pool;
  c.pool_r = p.pool_k / 2;
  c.n = p.n;
  c.base = p.base;
  c.sink_end = min(static_cast<int64_t>(p.n_sink), p.n_total);
  c.rec_begin = max(c.sink_end, p.n_total - static_cast<int64_t>(p.n_recent));
  c.slot_map = p.slot_map;
  c.dead = p.dead_slot;
  c.c0 = (p.cand_count != nullptr) ? min(max(p.cand_count[u], 0), p.k_total) : 0;
  const int kcap = p.k_total;
  uint32_t* ckey = dyn;
  int32_t* cidx = reinterpret_cast<int32_t*>(dyn + (p.cand_count != nullptr ? kcap : 0));
  uint32_t* tkey = dyn + (p.cand_count != nullptr ? 2 * kcap : 0);
  c.ckey = ckey;
  c.cidx = cidx;
  c.tkey = (MODE == kLdsKeys) ? tkey : (MODE == kPrepared) ? prep_keys + static_cast<int64_t>(u) * p.n : nullptr;

  // ---- alive forced positions of the whole unit
  uint32_t fs = 0, fr = 0;
  for (int64_t g = tid; g < c.sink_end; g += kThreads) fs += alive_at(c, g) ? 1u : 0u;
  for (int64_t g = c.rec_begin + tid; g < p.n_total; g += kThreads) fr += alive_at(c, g) ? 1u : 0u;
  const uint32_t fsum = block_sum(fs, sh.wave_cnt);
  const uint32_t rsum = block_sum(fr, sh.wave_cnt);
  const int32_t room = p.k_total - static_cast<int32_t>(fsum + rsum);

  // ---- stage running candidates and (optionally) this tile's keys in LDS
  for (int e = tid; e < c.c0; e += kThreads) {
    const int64_t o = static_cast<int64_t>(u) * kcap + e;
    ckey[e] = score_key(p.cand_score[o]);
    cidx[e] = p.cand_idx[o];
  }
  if constexpr (MODE == kLdsKeys) {
    for (int64_t j = tid; j < c.n; j += kThreads) {
      const int64_t g = c.base + j;
      tkey[j] = (forced_at(c, g) || !alive_at(c, g)) ? 0u : score_key(column_score(c, j));
    }
  }
  __syncthreads();

  const int64_t M = c.c0 + c.n;
  uint32_t cc = 0;
  if constexpr (MODE == kPrepared) {
    // the first radix pass: the slices' top-byte histograms summed in order,
    // plus the running candidates' top bytes
    for (int b = tid; b < 256; b += kThreads) {
      uint32_t t = 0;
      for (int sl = 0; sl < n_slices; ++sl) t += prep_hist[(static_cast<int64_t>(u) * n_slices + sl) * 256 + b];
      sh.hist[b] = t;
      cc += t;
    }
    __syncthreads();
    for (int e = tid; e < c.c0; e += kThreads) {
      const uint32_t key = ckey[e];
      if (key != 0u) {
        atomicAdd(&sh.hist[key >> 24], 1u);
        ++cc;
      }
    }
  } else {
    for (int64_t e = tid; e < M; e += kThreads) {
      int64_t g;
      cc += entry_key(c, e, &g) != 0u ? 1u : 0u;
    }
  }
  const uint32_t n_cand = block_sum(cc, sh.wave_cnt);

  // ---- radix select of the room-th largest key
  uint32_t T;
  int32_t remaining;
  if (static_cast<int64_t>(n_cand) <= static_cast<int64_t>(room)) {
    T = 1u;                 // no finite score maps to key 1: every candidate is "> T"
    remaining = 0;
  } else if (room <= 0) {
    T = 0xFFFFFFFFu;        // no finite score maps to this key: nothing is selected
    remaining = 0;
  } else {
    if (tid == 0) {
      sh.prefix = 0u;
      sh.remaining = room;
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hi_mask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
      const uint32_t prefix = sh.prefix;
      if (MODE != kPrepared || shift != 24) {       // prepared: the top-byte histogram is summed above
        __syncthreads();
        for (int b = tid; b < 256; b += kThreads) sh.hist[b] = 0u;
        __syncthreads();
        if constexpr (MODE == kPrepared) {
          // candidates from LDS, tile keys from the workspace four at a time
          for (int e = tid; e < c.c0; e += kThreads) {
            const uint32_t key = ckey[e];
            if (key != 0u && ((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
          }
          for (int64_t j0 = tid; j0 < c.n; j0 += 4 * kThreads) {
            uint32_t kq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) kq[q] = (j0 + q * kThreads < c.n) ? c.tkey[j0 + q * kThreads] : 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (kq[q] != 0u && ((kq[q] ^ prefix) & hi_mask) == 0u)
                atomicAdd(&sh.hist[(kq[q] >> shift) & 255u], 1u);
          }
        } else {
          for (int64_t e = tid; e < M; e += kThreads) {
            int64_t g;
            const uint32_t key = entry_key(c, e, &g);
            if (key != 0u && ((key ^ prefix) & hi_mask) == 0u)
              atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wave == 0) find_bin(sh, prefix, shift, lane);
      __syncthreads();
    }
    T = sh.prefix;
    remaining = sh.remaining;
  }

  // ---- sweep A: per-wave counts of keys == T and > T over contiguous segments
  const int64_t seg = ((M + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t s_beg = min(M, static_cast<int64_t>(wave) * seg);
  const int64_t s_end = min(M, s_beg + seg);
  uint32_t n_eq = 0, n_gt = 0;
  for (int64_t e0 = s_beg; e0 < s_end; e0 += 4 * 64) {
    uint32_t kq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t e = e0 + 64 * q + lane;
      kq[q] = 0u;
      if (e < s_end) {
        int64_t g;
        kq[q] = entry_key(c, e, &g);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      n_eq += __popcll(__ballot(kq[q] != 0u && kq[q] == T));
      n_gt += __popcll(__ballot(kq[q] != 0u && kq[q] > T));
    }
  }
  if (lane == 0) {
    sh.wave_eq[wave] = n_eq;
    sh.wave_gt[wave] = n_gt;
  }
  __syncthreads();
  uint32_t eq_base = 0, sel_base = 0;
  for (int w = 0; w < wave; ++w) {
    const int32_t take_eq = max(0, min(static_cast<int32_t>(sh.wave_eq[w]),
                                       remaining - static_cast<int32_t>(eq_base)));
    sel_base += sh.wave_gt[w] + static_cast<uint32_t>(take_eq);
    eq_base += sh.wave_eq[w];
  }
  uint32_t n_sel_total = 0;
  {
    uint32_t eb = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int32_t take_eq = max(0, min(static_cast<int32_t>(sh.wave_eq[w]),
                                         remaining - static_cast<int32_t>(eb)));
      n_sel_total += sh.wave_gt[w] + static_cast<uint32_t>(take_eq);
      eb += sh.wave_eq[w];
    }
  }

  // ---- sweep B: place the selected entries in ascending index order
  const int64_t sink_alive = static_cast<int64_t>(fsum);
  const bool untiled_mask = p.finalize && p.keep_mask != nullptr;
  int32_t* kept = p.kept_idx + static_cast<int64_t>(u) * p.k_total;
  for (int64_t e00 = s_beg; e00 < s_end; e00 += 4 * 64) {
   uint32_t kq[4];
   int64_t gq[4];
#pragma unroll
   for (int q = 0; q < 4; ++q) {
     const int64_t e = e00 + 64 * q + lane;
     kq[q] = 0u;
     gq[q] = -1;
     if (e < s_end) kq[q] = entry_key(c, e, &gq[q]);
   }
#pragma unroll
   for (int q = 0; q < 4; ++q) {
    const int64_t e = e00 + 64 * q + lane;
    const uint32_t key = kq[q];
    const int64_t g = gq[q];
    const bool is_eq = key != 0u && key == T;
    const bool is_gt = key != 0u && key > T;
    const uint64_t beq = __ballot(is_eq);
    const uint32_t eq_rank = eq_base + __popcll(beq & lanemask_lt(lane));
    const bool sel = is_gt || (is_eq && static_cast<int32_t>(eq_rank) < remaining);
    const uint64_t bsel = __ballot(sel);
    const uint32_t pos = sel_base + __popcll(bsel & lanemask_lt(lane));
    if (sel) {
      if (p.finalize) {
        kept[sink_alive + pos] = static_cast<int32_t>(g);
      } else {
        const int64_t o = static_cast<int64_t>(u) * p.k_total + pos;
        p.cand_score[o] = key_score(key);
        p.cand_idx[o] = static_cast<int32_t>(g);
      }
    }
    if (untiled_mask && e < s_end) {
      const bool keep = sel || (forced_at(c, g) && alive_at(c, g));
      p.keep_mask[static_cast<int64_t>(u) * p.n_total + g] = keep ? 1 : 0;
    }
    eq_base += __popcll(beq);
    sel_base += __popcll(bsel);
   }
  }

  if (!p.finalize) {
    if (tid == 0) p.cand_count[u] = static_cast<int32_t>(n_sel_total);
    return;
  }

  // ---- forced entries: alive sink first, alive recent last
  if (wave == 0) {
    uint32_t r = 0;
    for (int64_t g0 = 0; g0 < c.sink_end; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < c.sink_end && alive_at(c, g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  } else if (wave == 1) {
    uint32_t r = static_cast<uint32_t>(sink_alive) + n_sel_total;
    for (int64_t g0 = c.rec_begin; g0 < p.n_total; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < p.n_total && alive_at(c, g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  }
  const int64_t total = sink_alive + n_sel_total + rsum;
  for (int64_t i = total + tid; i < p.k_total; i += kThreads) kept[i] = -1;
  if (tid == 0 && p.n_kept != nullptr) p.n_kept[u] = static_cast<int32_t>(total);
}

// Per-unit selection over keys held in registers.  Wavefront w owns the
// contiguous segment [w*seg, (w+1)*seg) of the unit in rows of 64 columns
// (KPT rows), so the ballot sweeps see columns in ascending order.  Requires
// n <= KPT * NT (NT threads per workgroup: 1024, or 256 for short rows,
// whose barriers then wait on 4 wavefronts instead of 16).  With kFused (unpooled calls) the keys are made here
// from the score row and the first radix pass runs here too; otherwise they
// come prepared, with the slices' top-byte histograms, from
// select_keys_kernel.
// Max pooling of radius R over a wavefront's columns held in registers:
// v[i] on lane l is column s_beg + 64 i + l.  The chunks are extended by the
// 64 columns before and after them (b[0] and b[KPT + 1], loaded here);
// columns outside the row count as -inf, so every window takes the maximum
// of its in-range columns.  With P the largest power of two not above the
// window 2R + 1, log2(P) doubling steps give b[c] = max of columns
// [c, c + P), and the window of c is max(b[c - R], b[c + R + 1 - P]).  A
// shift by d columns moves every chunk's values by one lane shuffle; lanes
// that cross a chunk edge take the neighbouring chunk's shuffled values.
template <int KPT>
__device__ __forceinline__ void pool_max_regs(float (&v)[KPT], const float* row, int n, int s_beg, int lane,
                                              int R) {
  constexpr int C = KPT + 2;
  const int P = (2 * R + 1 >= 8) ? 8 : (2 * R + 1 >= 4) ? 4 : 2;   // R in [1, 7]
  const float kNegInf = -__builtin_huge_valf();
  float b[C];
  const int el = s_beg - 64 + lane, er = s_beg + 64 * KPT + lane;
  const float fl = row[min(max(el, 0), n - 1)], fr = row[min(er, n - 1)];
  b[0] = (el >= 0 && el < n) ? fl : kNegInf;
#pragma unroll
  for (int i = 0; i < KPT; ++i) b[i + 1] = (s_beg + 64 * i + lane < n) ? v[i] : kNegInf;
  b[C - 1] = (er < n) ? fr : kNegInf;
  for (int m = 1; m < P; m <<= 1) {                 // b[c] = max over [c, c + 2m)
    const int src = (lane + m) & 63;
    const bool wrap = lane + m >= 64;
    // ascending: chunk j + 1 is shuffled before it is updated
    float cur = __shfl(b[0], src, 64);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float nxt = (j + 1 < C) ? __shfl(b[j + 1], src, 64) : kNegInf;
      b[j] = fmaxf(b[j], wrap ? nxt : cur);
      cur = nxt;
    }
  }
  // v[i] = max(b at c - R, b at c + R + 1 - P): both offsets are <= 0
  const int d1 = -R, d2 = R + 1 - P;
  const int src1 = (lane + d1) & 63, src2 = (lane + d2) & 63;
  const bool wrap1 = lane + d1 < 0, wrap2 = lane + d2 < 0;
  float p1 = __shfl(b[0], src1, 64);
  float p2 = (d2 == 0) ? b[0] : __shfl(b[0], src2, 64);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const float c1 = __shfl(b[i + 1], src1, 64);
    const float c2 = (d2 == 0) ? b[i + 1] : __shfl(b[i + 1], src2, 64);
    v[i] = fmaxf(wrap1 ? p1 : c1, wrap2 ? p2 : c2);
    p1 = c1;
    p2 = c2;
  }
}

// Average pooling of radius R over the same register layout: each column's
// window is summed from 0 in ascending column order, columns outside the row
// counting as 0, then divided by 2R + 1 (the order the key preparation uses,
// so the pooled values are the same bits).  One shift per window offset.
template <int KPT>
__device__ __forceinline__ void pool_avg_regs(float (&v)[KPT], const float* row, int n, int s_beg, int lane,
                                              int R) {
  constexpr int C = KPT + 2;
  float b[C];
  const int el = s_beg - 64 + lane, er = s_beg + 64 * KPT + lane;
  const float fl = row[min(max(el, 0), n - 1)], fr = row[min(er, n - 1)];
  b[0] = (el >= 0 && el < n) ? fl : 0.f;
#pragma unroll
  for (int i = 0; i < KPT; ++i) b[i + 1] = (s_beg + 64 * i + lane < n) ? v[i] : 0.f;
  b[C - 1] = (er < n) ? fr : 0.f;
  float acc[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) acc[i] = 0.f;
  for (int d = -R; d <= R; ++d) {
    const int src = (lane + d) & 63;
    if (d == 0) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) acc[i] += b[i + 1];
    } else if (d < 0) {
      const bool wrap = lane + d < 0;                // from the chunk before
      float prev = __shfl(b[0], src, 64);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const float cur = __shfl(b[i + 1], src, 64);
        acc[i] += wrap ? prev : cur;
        prev = cur;
      }
    } else {
      const bool wrap = lane + d >= 64;              // from the chunk after
      float cur = __shfl(b[1], src, 64);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const float nxt = __shfl(b[i + 2], src, 64);
        acc[i] += wrap ? nxt : cur;
        cur = nxt;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) v[i] = acc[i] / static_cast<float>(2 * R + 1);
}

template <int KPT, bool kFused, int NT>
__global__ __launch_bounds__(NT) void select_regs_kernel(SelectParams p, const float* scores,
                                                               const uint32_t* keys,
                                                               const uint32_t* hist, int n_slices) {
  constexpr int NW = NT / 64;
  __shared__ SelShared sh;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = static_cast<int>(p.n);              // untiled: n == n_total, base == 0
  const int sink_end = static_cast<int>(min(static_cast<int64_t>(p.n_sink), p.n_total));
  const int rec_begin = static_cast<int>(max(static_cast<int64_t>(sink_end), p.n_total - p.n_recent));
  auto alive = [&](int g) {
    return p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[g]) != p.dead_slot;
  };

  // ---- alive forced positions, top-byte histogram, candidate count
  uint32_t fs = 0, fr = 0, cc = 0;
  for (int g = tid; g < sink_end; g += NT) fs += alive(g) ? 1u : 0u;
  for (int g = rec_begin + tid; g < n; g += NT) fr += alive(g) ? 1u : 0u;
  const int seg = ((n + NW - 1) / NW + 63) / 64 * 64;
  const int s_beg = min(n, wave * seg);
  const int s_end = min(n, s_beg + seg);
  uint32_t kr[KPT];
  if constexpr (!kFused) {
    for (int b = tid; b < 256; b += NT) {
      uint32_t t = 0;
      for (int sl = 0; sl < n_slices; ++sl) t += hist[(static_cast<int64_t>(u) * n_slices + sl) * 256 + b];
      sh.hist[b] = t;
      cc += t;
    }
    // this wavefront's keys (0 past the segment)
    const uint32_t* ku = keys + static_cast<int64_t>(u) * n;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = s_beg + 64 * i + lane;
      kr[i] = (e < s_end) ? ku[e] : 0u;
    }
  } else {
    for (int b = tid; b < 256; b += NT) sh.hist[b] = 0u;
    const float* row = scores + static_cast<int64_t>(u) * p.row_stride;
    // unconditional loads (a clamped column past the segment) keep all KPT
    // in flight; a conditional load would wait for each one in turn
    float v[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = row[min(s_beg + 64 * i + lane, n - 1)];
    // pooling on the registers: max windows of radius 1 .. kFusedMaxPoolR;
    // average windows of that radius on rows of at most 8 keys per thread
    if (p.pool == KVSEL_POOL_MAX && p.pool_k > 1) {
      pool_max_regs<KPT>(v, row, n, s_beg, lane, p.pool_k / 2);
    } else if constexpr (KPT <= kFusedAvgKpt) {
      if (p.pool == KVSEL_POOL_AVG && p.pool_k > 1) pool_avg_regs<KPT>(v, row, n, s_beg, lane, p.pool_k / 2);
    }
    __syncthreads();                                // histogram cleared
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = s_beg + 64 * i + lane;
      uint32_t key = 0u;
      if (e < s_end && e >= sink_end && e < rec_begin) {   // no slot map on this path
        key = score_key(v[i]);
        atomicAdd(&sh.hist[key >> 24], 1u);
        ++cc;
      }
      kr[i] = key;
    }
  }
  const uint3 sums = block_sum3(fs, fr, cc, sh.wave_sums, NW);
  const uint32_t fsum = sums.x, rsum = sums.y, n_cand = sums.z;
  const int32_t room = p.k_total - static_cast<int32_t>(fsum + rsum);

  // ---- radix select of the room-th largest key (top byte already counted)
  uint32_t T;
  int32_t remaining;
  if (static_cast<int64_t>(n_cand) <= static_cast<int64_t>(room)) {
    T = 1u;                 // no finite score maps to key 1: every candidate is "> T"
    remaining = 0;
  } else if (room <= 0) {
    T = 0xFFFFFFFFu;        // no finite score maps to this key: nothing is selected
    remaining = 0;
  } else {
    if (tid == 0) {
      sh.prefix = 0u;
      sh.remaining = room;
    }
    __syncthreads();
    if (wave == 0) find_bin(sh, 0u, 24, lane);
    __syncthreads();
    for (int shift = 16; shift >= 0; shift -= 8) {
      const uint32_t hi_mask = 0xFFFFFFFFu << (shift + 8);
      const uint32_t prefix = sh.prefix;
      for (int b = tid; b < 256; b += NT) sh.hist[b] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t key = kr[i];
        if (key != 0u && ((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) find_bin(sh, prefix, shift, lane);
      __syncthreads();
    }
    T = sh.prefix;
    remaining = sh.remaining;
  }

  // ---- sweep A: per-wave counts of keys == T and > T
  uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t key = kr[i];
    n_eq += __popcll(__ballot(key != 0u && key == T));
    n_gt += __popcll(__ballot(key != 0u && key > T));
  }
  if (lane == 0) {
    sh.wave_eq[wave] = n_eq;
    sh.wave_gt[wave] = n_gt;
  }
  __syncthreads();
  uint32_t eq_base = 0, sel_base = 0, n_sel_total = 0;
  {
    uint32_t eb = 0;
    for (int w = 0; w < NW; ++w) {
      const int32_t take_eq = max(0, min(static_cast<int32_t>(sh.wave_eq[w]), remaining - static_cast<int32_t>(eb)));
      if (w == wave) {
        eq_base = eb;
        sel_base = n_sel_total;
      }
      n_sel_total += sh.wave_gt[w] + static_cast<uint32_t>(take_eq);
      eb += sh.wave_eq[w];
    }
  }

  // ---- sweep B: place the selected entries in ascending index order
  int32_t* kept = p.kept_idx + static_cast<int64_t>(u) * p.k_total;
  uint8_t* mask = (p.keep_mask != nullptr) ? p.keep_mask + static_cast<int64_t>(u) * p.n_total : nullptr;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int e = s_beg + 64 * i + lane;
    const uint32_t key = kr[i];
    const bool is_eq = key != 0u && key == T;
    const bool is_gt = key != 0u && key > T;
    const uint64_t beq = __ballot(is_eq);
    const uint32_t eq_rank = eq_base + __popcll(beq & lanemask_lt(lane));
    const bool sel = is_gt || (is_eq && static_cast<int32_t>(eq_rank) < remaining);
    const uint64_t bsel = __ballot(sel);
    const uint32_t pos = sel_base + __popcll(bsel & lanemask_lt(lane));
    if (sel) kept[fsum + pos] = e;
    if (mask != nullptr && e < s_end) {
      const bool keep = sel || ((e < sink_end || e >= rec_begin) && alive(e));
      mask[e] = keep ? 1 : 0;
    }
    eq_base += __popcll(beq);
    sel_base += __popcll(bsel);
  }

  // ---- forced entries: alive sink first, alive recent last
  if (wave == 0) {
    uint32_t r = 0;
    for (int g0 = 0; g0 < sink_end; g0 += 64) {
      const int g = g0 + lane;
      const bool a = g < sink_end && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = g;
      r += __popcll(b);
    }
  } else if (wave == 1) {
    uint32_t r = fsum + n_sel_total;
    for (int g0 = rec_begin; g0 < n; g0 += 64) {
      const int g = g0 + lane;
      const bool a = g < n && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = g;
      r += __popcll(b);
    }
  }
  const int64_t total = static_cast<int64_t>(fsum) + n_sel_total + rsum;
  for (int64_t i = total + tid; i < p.k_total; i += NT) kept[i] = -1;
  if (tid == 0 && p.n_kept != nullptr) p.n_kept[u] = static_cast<int32_t>(total);
}

// ---- few units of long untiled rows: the radix passes spread over the
// 4096-column slices of select_keys_kernel, one launch per step.  Each
// digit launch sums the previous digit's per-slice histograms in slice
// order (every workgroup the same way, so all find the same bin), slice 0's
// workgroup records the state for the next launch, and every workgroup
// histograms the next digit over its own slice.  The count launch fixes the
// threshold key T and counts each slice's keys above and equal to it; the
// placement launch writes each slice's selected positions in ascending
// order after those of the slices before it (keys equal to T ranked by
// position across the whole row, as the single-workgroup sweeps do).
constexpr int kSliceMaxUnits = 8;     // units per call that take the slice-parallel path
constexpr int kSliceState = 8;        // ints per unit and step: prefix, remaining, mode, fsum, rsum

struct SliceWs {
  uint32_t* keys;       // [U][n]
  uint32_t* hist0;      // [U][slices][256] top byte (select_keys_kernel)
  uint32_t* hist[2];    // [U][slices][256] later digits, alternating
  int32_t* state;       // [4][U][kSliceState]
  uint32_t* counts;     // [U][slices][2]: keys above T, keys equal to T
};

// Alive forced positions of unit u (sink, recent); all threads call.
__device__ void slice_forced(const SelectParams& p, uint32_t* scratch, uint32_t* fsum, uint32_t* rsum) {
  const int64_t sink_end = min(static_cast<int64_t>(p.n_sink), p.n_total);
  const int64_t rec_begin = max(sink_end, p.n_total - static_cast<int64_t>(p.n_recent));
  uint32_t fs = 0, fr = 0;
  for (int64_t g = threadIdx.x; g < sink_end; g += kPrepThreads)
    fs += (p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[g]) != p.dead_slot) ? 1u : 0u;
  for (int64_t g = rec_begin + threadIdx.x; g < p.n_total; g += kPrepThreads)
    fr += (p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[g]) != p.dead_slot) ? 1u : 0u;
  const uint3 t = block_sum3(fs, fr, 0u, scratch, kPrepThreads / 64);
  *fsum = t.x;
  *rsum = t.y;
}

// Digit step `step` (1, 2, 3: histograms of the digits at 16, 8, 0 bits):
// find the bin of the previous digit from `hin`, then histogram this digit.
__global__ __launch_bounds__(kPrepThreads) void slice_digit_kernel(SelectParams p, SliceWs w, int n_slices,
                                                                   int step, const uint32_t* hin,
                                                                   uint32_t* hout) {
  __shared__ SelShared sh;
  const int u = blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* st_out = w.state + (static_cast<int64_t>(step - 1) * p.U + u) * kSliceState;
  uint32_t prefix, fsum, rsum;
  int32_t rem, mode;
  // the summed histogram of the previous digit, slices in order
  uint32_t nc = 0;
  for (int b = tid; b < 256; b += kPrepThreads) {
    uint32_t t = 0;
    for (int sl = 0; sl < n_slices; ++sl) t += hin[(static_cast<int64_t>(u) * n_slices + sl) * 256 + b];
    sh.hist[b] = t;
    nc += t;
  }
  if (step == 1) {
    slice_forced(p, sh.wave_sums, &fsum, &rsum);
    const uint32_t n_cand = block_sum3(nc, 0u, 0u, sh.wave_sums, kPrepThreads / 64).x;
    const int32_t room = p.k_total - static_cast<int32_t>(fsum + rsum);
    prefix = 0u;
    rem = room;
    mode = (static_cast<int64_t>(n_cand) <= static_cast<int64_t>(room)) ? 1 : (room <= 0) ? 2 : 0;
  } else {
    const int32_t* st_in = w.state + (static_cast<int64_t>(step - 2) * p.U + u) * kSliceState;
    prefix = static_cast<uint32_t>(st_in[0]);
    rem = st_in[1];
    mode = st_in[2];
    fsum = static_cast<uint32_t>(st_in[3]);
    rsum = static_cast<uint32_t>(st_in[4]);
  }
  const int shift_in = 32 - 8 * step;          // the digit hin counts: 24, 16, 8
  if (mode == 0) {                              // uniform over the workgroup
    if (tid == 0) {
      sh.prefix = prefix;
      sh.remaining = rem;
    }
    __syncthreads();
    if (wave == 0) find_bin(sh, prefix, shift_in, lane);
    __syncthreads();
    prefix = sh.prefix;
    rem = sh.remaining;
  }
  if (slice == 0 && tid == 0) {
    st_out[0] = static_cast<int32_t>(prefix);
    st_out[1] = rem;
    st_out[2] = mode;
    st_out[3] = static_cast<int32_t>(fsum);
    st_out[4] = static_cast<int32_t>(rsum);
  }
  if (hout == nullptr) return;                  // the count launch reads the state itself
  // histogram of the next digit over this slice's keys that match the prefix
  const int shift = shift_in - 8;
  __syncthreads();
  for (int b = tid; b < 256; b += kPrepThreads) sh.hist[b] = 0u;
  __syncthreads();
  if (mode == 0) {
    const uint32_t hi_mask = 0xFFFFFFFFu << (shift + 8);
    const int64_t j0 = static_cast<int64_t>(slice) * kPrepKeys;
    const int jn = static_cast<int>(min(static_cast<int64_t>(kPrepKeys), p.n - j0));
    const uint32_t* ks = w.keys + static_cast<int64_t>(u) * p.n + j0;
    for (int i = tid; i < jn; i += kPrepThreads) {
      const uint32_t key = ks[i];
      if (key != 0u && ((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  uint32_t* ho = hout + (static_cast<int64_t>(u) * n_slices + slice) * 256;
  for (int b = tid; b < 256; b += kPrepThreads) ho[b] = sh.hist[b];
}

// The last digit's bin (from `hin`, the digit at 0 bits), the threshold key
// T, and each slice's keys above and equal to T.
__global__ __launch_bounds__(kPrepThreads) void slice_count_kernel(SelectParams p, SliceWs w, int n_slices,
                                                                   const uint32_t* hin) {
  __shared__ SelShared sh;
  const int u = blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* st_in = w.state + (static_cast<int64_t>(2) * p.U + u) * kSliceState;
  int32_t* st_out = w.state + (static_cast<int64_t>(3) * p.U + u) * kSliceState;
  uint32_t prefix = static_cast<uint32_t>(st_in[0]);
  int32_t rem = st_in[1];
  const int32_t mode = st_in[2];
  if (mode == 0) {
    for (int b = tid; b < 256; b += kPrepThreads) {
      uint32_t t = 0;
      for (int sl = 0; sl < n_slices; ++sl) t += hin[(static_cast<int64_t>(u) * n_slices + sl) * 256 + b];
      sh.hist[b] = t;
    }
    if (tid == 0) {
      sh.prefix = prefix;
      sh.remaining = rem;
    }
    __syncthreads();
    if (wave == 0) find_bin(sh, prefix, 0, lane);
    __syncthreads();
    prefix = sh.prefix;
    rem = sh.remaining;
  }
  // T as the single-workgroup select sets it: 1 (every candidate is above)
  // or 0xFFFFFFFF (nothing is selected) outside the radix case
  const uint32_t T = (mode == 1) ? 1u : (mode == 2) ? 0xFFFFFFFFu : prefix;
  if (mode != 0) rem = 0;
  if (slice == 0 && tid == 0) {
    st_out[0] = static_cast<int32_t>(T);
    st_out[1] = rem;
    st_out[2] = mode;
    st_out[3] = st_in[3];
    st_out[4] = st_in[4];
  }
  const int64_t j0 = static_cast<int64_t>(slice) * kPrepKeys;
  const int jn = static_cast<int>(min(static_cast<int64_t>(kPrepKeys), p.n - j0));
  const uint32_t* ks = w.keys + static_cast<int64_t>(u) * p.n + j0;
  uint32_t gt = 0, eq = 0;
  for (int i = tid; i < jn; i += kPrepThreads) {
    const uint32_t key = ks[i];
    gt += (key != 0u && key > T) ? 1u : 0u;
    eq += (key != 0u && key == T) ? 1u : 0u;
  }
  const uint3 t = block_sum3(gt, eq, 0u, sh.wave_sums, kPrepThreads / 64);
  if (tid == 0) {
    uint32_t* c = w.counts + (static_cast<int64_t>(u) * n_slices + slice) * 2;
    c[0] = t.x;
    c[1] = t.y;
  }
}

// Places the selected positions of one slice, writes its keep mask; slice
// 0's workgroup also places the forced positions and pads the list.
__global__ __launch_bounds__(kPrepThreads) void slice_place_kernel(SelectParams p, SliceWs w, int n_slices) {
  __shared__ SelShared sh;
  constexpr int kW = kPrepThreads / 64;
  const int u = blockIdx.y, slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* st = w.state + (static_cast<int64_t>(3) * p.U + u) * kSliceState;
  const uint32_t T = static_cast<uint32_t>(st[0]);
  const int32_t remaining = st[1];
  const uint32_t fsum = static_cast<uint32_t>(st[3]), rsum = static_cast<uint32_t>(st[4]);
  // bases from the slices before this one, and the total selected
  const uint32_t* cu = w.counts + static_cast<int64_t>(u) * n_slices * 2;
  uint32_t eq_base = 0, sel_base = 0, n_sel_total = 0, eb = 0;
  for (int sl = 0; sl < n_slices; ++sl) {
    const uint32_t g = cu[2 * sl], e = cu[2 * sl + 1];
    const int32_t take = max(0, min(static_cast<int32_t>(e), remaining - static_cast<int32_t>(eb)));
    if (sl < slice) {
      eq_base += e;
      sel_base += g + static_cast<uint32_t>(take);
    }
    n_sel_total += g + static_cast<uint32_t>(take);
    eb += e;
  }
  const int64_t sink_end = min(static_cast<int64_t>(p.n_sink), p.n_total);
  const int64_t rec_begin = max(sink_end, p.n_total - static_cast<int64_t>(p.n_recent));
  auto alive = [&](int64_t g) {
    return p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[g]) != p.dead_slot;
  };
  // wavefront segments of the slice, in order: counts, then bases
  const int64_t j0 = static_cast<int64_t>(slice) * kPrepKeys;
  const int jn = static_cast<int>(min(static_cast<int64_t>(kPrepKeys), p.n - j0));
  const int seg = kPrepKeys / kW;
  const int s_beg = min(jn, wave * seg), s_end = min(jn, s_beg + seg);
  const uint32_t* ks = w.keys + static_cast<int64_t>(u) * p.n + j0;
  uint32_t n_eq = 0, n_gt = 0;
  for (int i0 = s_beg; i0 < s_end; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t key = (i < s_end) ? ks[i] : 0u;
    n_eq += __popcll(__ballot(key != 0u && key == T));
    n_gt += __popcll(__ballot(key != 0u && key > T));
  }
  if (lane == 0) {
    sh.wave_eq[wave] = n_eq;
    sh.wave_gt[wave] = n_gt;
  }
  __syncthreads();
  for (int v = 0; v < wave; ++v) {
    const int32_t take = max(0, min(static_cast<int32_t>(sh.wave_eq[v]), remaining - static_cast<int32_t>(eq_base)));
    sel_base += sh.wave_gt[v] + static_cast<uint32_t>(take);
    eq_base += sh.wave_eq[v];
  }
  int32_t* kept = p.kept_idx + static_cast<int64_t>(u) * p.k_total;
  uint8_t* mask = (p.keep_mask != nullptr) ? p.keep_mask + static_cast<int64_t>(u) * p.n_total : nullptr;
  for (int i0 = s_beg; i0 < s_end; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t key = (i < s_end) ? ks[i] : 0u;
    const bool is_eq = key != 0u && key == T;
    const bool is_gt = key != 0u && key > T;
    const uint64_t beq = __ballot(is_eq);
    const uint32_t eq_rank = eq_base + __popcll(beq & lanemask_lt(lane));
    const bool sel = is_gt || (is_eq && static_cast<int32_t>(eq_rank) < remaining);
    const uint64_t bsel = __ballot(sel);
    const uint32_t pos = sel_base + __popcll(bsel & lanemask_lt(lane));
    const int64_t g = j0 + i;
    if (sel) kept[fsum + pos] = static_cast<int32_t>(g);
    if (mask != nullptr && i < s_end) {
      const bool forced = g < sink_end || g >= rec_begin;
      mask[g] = (sel || (forced && alive(g))) ? 1 : 0;
    }
    eq_base += __popcll(beq);
    sel_base += __popcll(bsel);
  }
  if (slice != 0) return;
  // forced entries: alive sink first, alive recent after the selected ones
  if (wave == 0) {
    uint32_t r = 0;
    for (int64_t g0 = 0; g0 < sink_end; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < sink_end && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  } else if (wave == 1) {
    uint32_t r = fsum + n_sel_total;
    for (int64_t g0 = rec_begin; g0 < p.n_total; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < p.n_total && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  }
  const int64_t total = static_cast<int64_t>(fsum) + n_sel_total + rsum;
  for (int64_t i = total + tid; i < p.k_total; i += kPrepThreads) kept[i] = -1;
  if (tid == 0 && p.n_kept != nullptr) p.n_kept[u] = static_cast<int32_t>(total);
}

static bool select_slice_path(const SelectParams& p) {
  return p.cand_count == nullptr && p.U <= kSliceMaxUnits && p.n > 32 * kThreads;
}

// Untiled calls without a slot map, with rows that fit the registers and
// either enough units to fill the device or rows short enough that one
// workgroup reads them at once, run select_regs_kernel alone when they are
// unpooled or their window is short (max up to 9; average up to 9 on rows
// of at most 2048, summed in the definition's order): each unit's
// workgroup pools and makes its keys from the scores, so no workspace is
// used (and a short call saves the second launch's latency).  Longer
// windows keep the two launches, whose key kernel stages the window's halo
// in LDS.  An empty row (n = 0, scores possibly NULL) takes the two-launch
// path, whose per-unit kernel reads no key when n is 0.
static bool select_single_launch(const SelectParams& p) {
  return p.cand_count == nullptr && p.n > 0 && p.n <= 32 * kThreads && (p.U >= kFusedMinUnits || p.n <= kFusedSmallN) &&
         (p.pool == KVSEL_POOL_NONE || p.pool_k == 1 || (p.pool == KVSEL_POOL_MAX && p.pool_k / 2 <= kFusedMaxPoolR) ||
          (p.pool == KVSEL_POOL_AVG && p.pool_k / 2 <= kFusedMaxPoolR && p.n <= kFusedAvgKpt * 256)) &&
         p.slot_map == nullptr;
}

// Bytes of the slice-parallel path's buffers after the keys and the top-byte
// histograms: two more digit histograms, the per-step state and the counts.
static int64_t slice_extra_bytes(const SelectParams& p, int64_t slices) {
  const int64_t hist = (static_cast<int64_t>(p.U) * slices * 256 * 4 + 255) / 256 * 256;
  const int64_t state = (static_cast<int64_t>(4) * p.U * kSliceState * 4 + 255) / 256 * 256;
  const int64_t counts = (static_cast<int64_t>(p.U) * slices * 2 * 4 + 255) / 256 * 256;
  return 2 * hist + state + counts;
}

size_t select_workspace_bytes(const SelectParams& p) {
  if (p.U == 0 || p.n == 0 || select_single_launch(p) || select_tile_fits(p)) return 0;
  const int64_t slices = ceil_div(p.n, kPrepKeys);
  const int64_t key_bytes = (static_cast<int64_t>(p.U) * p.n * 4 + 255) / 256 * 256;
  const int64_t hist0 = (static_cast<int64_t>(p.U) * slices * 256 * 4 + 255) / 256 * 256;
  return static_cast<size_t>(key_bytes + hist0 + (select_slice_path(p) ? slice_extra_bytes(p, slices) : 0));
}

hipError_t launch_select(const SelectParams& p, const float* scores, void* ws, hipStream_t st) {
  if (p.U == 0) return hipSuccess;
  const bool tiled = p.cand_count != nullptr;
  if (!tiled) {
    uint32_t* keys = static_cast<uint32_t*>(ws);
    const int n_slices = static_cast<int>(ceil_div(p.n, kPrepKeys));
    uint32_t* hist = keys + (static_cast<int64_t>(p.U) * p.n * 4 + 255) / 256 * 64;
    if (select_single_launch(p)) {
      static_assert(kFusedAvgKpt == 8, "average windows run on the 8-keys-per-thread kernel only");
      if (p.n <= 8 * 256) select_regs_kernel<8, true, 256><<<p.U, 256, 0, st>>>(p, scores, nullptr, nullptr, 0);
      else select_regs_kernel<32, true, kThreads><<<p.U, kThreads, 0, st>>>(p, scores, nullptr, nullptr, 0);
      return hipGetLastError();
    }
    if (n_slices > 0) {
      dim3 grid(n_slices, p.U);
      select_keys_kernel<<<grid, kPrepThreads, 0, st>>>(p, scores, keys, hist);
    }
    if (select_slice_path(p)) {
      // few units of long rows: the remaining radix steps spread over the slices
      uint8_t* base = reinterpret_cast<uint8_t*>(hist) +
                      (static_cast<int64_t>(p.U) * n_slices * 256 * 4 + 255) / 256 * 256;
      const int64_t hb = (static_cast<int64_t>(p.U) * n_slices * 256 * 4 + 255) / 256 * 256;
      const int64_t sb = (static_cast<int64_t>(4) * p.U * kSliceState * 4 + 255) / 256 * 256;
      SliceWs w;
      w.keys = keys;
      w.hist0 = hist;
      w.hist[0] = reinterpret_cast<uint32_t*>(base);
      w.hist[1] = reinterpret_cast<uint32_t*>(base + hb);
      w.state = reinterpret_cast<int32_t*>(base + 2 * hb);
      w.counts = reinterpret_cast<uint32_t*>(base + 2 * hb + sb);
      dim3 grid(n_slices, p.U);
      slice_digit_kernel<<<grid, kPrepThreads, 0, st>>>(p, w, n_slices, 1, w.hist0, w.hist[0]);
      slice_digit_kernel<<<grid, kPrepThreads, 0, st>>>(p, w, n_slices, 2, w.hist[0], w.hist[1]);
      slice_digit_kernel<<<grid, kPrepThreads, 0, st>>>(p, w, n_slices, 3, w.hist[1], w.hist[0]);
      slice_count_kernel<<<grid, kPrepThreads, 0, st>>>(p, w, n_slices, w.hist[0]);
      slice_place_kernel<<<grid, kPrepThreads, 0, st>>>(p, w, n_slices);
      return hipGetLastError();
    }
    // up to 32 keys per thread stay in registers; larger units stream their
    // keys from the workspace (64 per thread no longer fit without spilling)
    if (p.n <= 32 * kThreads)
      select_regs_kernel<32, false, kThreads><<<p.U, kThreads, 0, st>>>(p, scores, keys, hist, n_slices);
    else
      select_kernel<kPrepared><<<p.U, kThreads, 0, st>>>(p, scores, keys, hist, n_slices);
    return hipGetLastError();
  }
  if (select_tile_fits(p)) return launch_select_tile(p, scores, st);
  const size_t cand_bytes = static_cast<size_t>(p.k_total) * 8;
  if (p.n > 0) {
    // tiled, prepared: keys and top-byte histograms of the tile, then the
    // per-unit merge with the running candidates staged in LDS
    uint32_t* keys = static_cast<uint32_t*>(ws);
    const int n_slices = static_cast<int>(ceil_div(p.n, kPrepKeys));
    uint32_t* hist = keys + (static_cast<int64_t>(p.U) * p.n * 4 + 255) / 256 * 64;
    dim3 grid(n_slices, p.U);
    select_keys_kernel<<<grid, kPrepThreads, 0, st>>>(p, scores, keys, hist);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<kPrepared>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(cand_bytes));
    if (e != hipSuccess) return e;
    select_kernel<kPrepared><<<p.U, kThreads, cand_bytes, st>>>(p, scores, keys, hist, n_slices);
    return hipGetLastError();
  }
  const bool lds_keys = p.n <= kLdsKeysMax && cand_bytes + static_cast<size_t>(p.n) * 4 <= 150 * 1024;
  const size_t shmem = cand_bytes + (lds_keys ? static_cast<size_t>(p.n) * 4 : 0);
  if (lds_keys) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<kLdsKeys>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(shmem));
    if (e != hipSuccess) return e;
    select_kernel<kLdsKeys><<<p.U, kThreads, shmem, st>>>(p, scores, nullptr, nullptr, 0);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<kOnTheFly>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(shmem));
    if (e != hipSuccess) return e;
    select_kernel<kOnTheFly><<<p.U, kThreads, shmem, st>>>(p, scores, nullptr, nullptr, 0);
  }
  return hipGetLastError();
}

}  // namespace kvsel
