// Tiled budgeted top-k: one tile of scores merged into running candidates.
//
// KVMem (query-conditioned retrieval) scores a large Mean-K index in bounded
// tiles; the selection over the whole index must equal the untiled one
// (IntentKV §4 top-k with the forced set, ties to the lower index, output
// in chronological order).  Each unit keeps its best `room` non-forced
// entries so far as running candidates, in ascending global index; a tile
// call merges the tile's columns into them.
//
// One workgroup per unit reads its tile row once.  When the running set is
// full, its smallest key T0 is a threshold no tile column at or below can
// pass (a tile column equal to T0 loses the tie to the earlier candidate),
// so only columns above T0 survive.  Survivors go to LDS (key, column) and
// a 12-bit histogram of their top key bits is built on the way.  The
// selection is a radix select over candidates + survivors with digits of 12,
// 12 and 8 bits.  If the survivors do not fit in LDS (the first tile, or an
// adversarial tile), the first digit's histogram bounds the threshold bin,
// and the tile is read again keeping only keys at or above that bin (or the
// second digit's bin); if even that does not fit, the remaining digits and
// the placement read the tile from global memory each time.
//
// A packed tile (the block scorer's output when given the running set's
// threshold) holds only the columns admitted above it: the same passes run
// over the admitted columns, read through the chunk masks.  A call that
// does not finalize can write that threshold for the next tile: the
// smallest score of the running set once it holds `room` entries, NaN
// (admit everything) before.
//
// Placement keeps ascending order without a sort: selected candidates come
// first (all their indices precede the tile), in array order by a block
// scan; selected tile columns are marked in a bitmap over the tile and
// placed by the rank of their bit.  Ties at the threshold key T go to the
// candidates first, then to the lowest tile columns (ranked by the same
// bitmap).
#include "common.h"

namespace kvsel {

namespace {

constexpr int kT = 1024;                 // threads per workgroup
constexpr int kW = kT / 64;
constexpr int kBins = 4096;              // 12-bit digits
constexpr int kMaxCandPerThread = 8;     // k_total <= 8192

struct TileShared {
  uint32_t hist[kBins];
  uint32_t scan[kT];                     // per-thread exclusive prefixes
  uint32_t wred[4 * kW];
  uint32_t n_surv;
  uint32_t bin, above, rem;
};

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
}

// Block-wide exclusive prefix over threads of v (and the total).  All threads call.
__device__ uint32_t block_exclusive(uint32_t v, TileShared& sh, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) sh.wred[wave] = incl;
  __syncthreads();
  // lane w < kW holds wave w's total: the sums over all waves and over the
  // waves before this one, by a butterfly over the first kW lanes (every
  // lane of the wavefront is active here), read from lane 0
  uint32_t all = (lane < kW) ? sh.wred[lane] : 0u;
  uint32_t before = (lane < wave) ? all : 0u;
#pragma unroll
  for (int o = kW / 2; o > 0; o >>= 1) {
    all += __shfl_xor(all, o, 64);
    before += __shfl_xor(before, o, 64);
  }
  all = __builtin_amdgcn_readfirstlane(all);
  before = __builtin_amdgcn_readfirstlane(before);
  *total = all;
  return before + incl - v;
}

__device__ uint32_t block_sum_u32(uint32_t v, TileShared& sh) {
  uint32_t total;
  block_exclusive(v, sh, &total);
  return total;
}

__device__ uint32_t block_min_u32(uint32_t v, TileShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(v, o, 64)));
  __syncthreads();
  if (lane == 0) sh.wred[wave] = v;
  __syncthreads();
  uint32_t m = (lane < kW) ? sh.wred[lane] : 0xFFFFFFFFu;
#pragma unroll
  for (int o = kW / 2; o > 0; o >>= 1) m = min(m, static_cast<uint32_t>(__shfl_xor(m, o, 64)));
  return __builtin_amdgcn_readfirstlane(m);
}

// Over sh.hist[0, nbins): the bin holding the rem-th largest entry, the count
// of entries in bins above it, and the updated rank within the bin.  All
// threads call; results in sh.bin / sh.above / sh.rem.
__device__ void find_bin_block(TileShared& sh, int nbins, uint32_t rem) {
  const int tid = threadIdx.x;
  const int per = nbins / kT > 0 ? nbins / kT : 1;       // bins per thread (4 or 1)
  const int b0 = tid * per;
  // thread tid owns bins [b0, b0 + per); count of bins above mine = suffix
  uint32_t own = 0;
  if (b0 < nbins)
    for (int i = 0; i < per; ++i) own += sh.hist[b0 + i];
  // suffix over threads = total - inclusive prefix
  uint32_t total;
  const uint32_t excl = block_exclusive(own, sh, &total);
  const uint32_t above_me = total - excl - own;
  if (b0 < nbins && above_me < rem && above_me + own >= rem) {
    uint32_t acc = above_me;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t h = sh.hist[b0 + i];
      if (acc + h >= rem) {
        sh.bin = static_cast<uint32_t>(b0 + i);
        sh.above = acc;
        sh.rem = rem - acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

struct Tile {
  const float* row;
  const uint64_t* mask;                  // packed tile: the row's admission masks; NULL: dense
  int n;                                 // columns of the tile; all positions are < 2^31
  int base, sink_end, rec_begin;
  const int32_t* slot_map;
  int64_t dead;
  bool vec;                              // row 16-byte aligned and n % 4 == 0
};

// Key of tile column j (0 = not a candidate: forced or dead).
__device__ __forceinline__ uint32_t tile_key(const Tile& t, int j, float s) {
  const int g = t.base + j;
  if (g < t.sink_end || g >= t.rec_begin) return 0u;
  if (t.slot_map != nullptr && static_cast<int64_t>(t.slot_map[g]) == t.dead) return 0u;
  return score_key(s);
}

// Key of tile column j of a tile without a slot map (in_row: j < n).
__device__ __forceinline__ uint32_t dense_key(const Tile& t, bool in_row, int j, float s) {
  const int g = t.base + j;
  return (in_row && g >= t.sink_end && g < t.rec_begin) ? score_key(s) : 0u;
}

constexpr int kDenseBatch = 4;           // float4 loads in flight per thread on dense tiles

// Calls f(j, key) for every tile column, key = 0 unless the column is a
// candidate with key >= lo (lo >= 1), reading the row from global memory.
// All lanes of a wavefront run the same number of iterations (f may use
// wave-wide operations); columns past the tile come with key 0.  A packed
// tile is visited one mask word per lane, over the word's set bits: an
// admitted column's score sits at the rank of its bit among the chunk's
// set bits.  Only admitted columns are visited; idle lanes call f with
// column -1 and key 0.
template <bool kPacked, bool kFast = true, typename F>
__device__ __forceinline__ void for_tile(const Tile& t, uint32_t lo, F&& f) {
  const int tid = threadIdx.x;
  if constexpr (kPacked) {
    // one lane per mask word (64 columns); the four lanes of a chunk's
    // words sit side by side, so a lane's first packed position is the
    // chunk start plus the popcounts of the lanes before it in its chunk
    const int lane = tid & 63;
    const int n_words = (t.n + 63) / 64;
    for (int wb = 0; wb < n_words; wb += kT) {
      const int w = wb + tid;
      uint64_t m = 0ull;
      if (w < n_words) {
        m = t.mask[w];
        const int rest = t.n - 64 * w;                  // bits past the tile are ignored
        if (rest < 64) m &= (1ull << rest) - 1ull;
      }
      const uint32_t pc = static_cast<uint32_t>(__popcll(m));
      const int q = lane & 3;                           // word within the chunk (kPackChunk = 4 words)
      const uint32_t p1 = __shfl_up(pc, 1, 64), p2 = __shfl_up(pc, 2, 64), p3 = __shfl_up(pc, 3, 64);
      int at = (w / 4) * kPackChunk + static_cast<int>((q >= 1 ? p1 : 0u) + (q >= 2 ? p2 : 0u) + (q >= 3 ? p3 : 0u));
      while (__ballot(m != 0ull) != 0ull) {             // uniform over the wavefront
        int col = -1;
        uint32_t key = 0u;
        if (m != 0ull) {
          const int b = __ffsll(static_cast<unsigned long long>(m)) - 1;
          m &= m - 1ull;
          col = 64 * w + b;
          key = tile_key(t, col, t.row[at]);
          ++at;
        }
        f(col, key >= lo ? key : 0u);
      }
    }
    return;
  }
  if (kFast && t.vec && t.slot_map == nullptr) {
    // no slot map: a column's key depends on its position and score only,
    // so it is formed without branches; the batch's loads are issued
    // together (past the row they repeat its last 16 bytes, unused)
    const float4* r4 = reinterpret_cast<const float4*>(t.row);
    const int n4 = t.n / 4;
    constexpr int kU = kDenseBatch;
    for (int ib = 0; ib < n4; ib += kU * kT) {
      float4 v[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) v[q] = r4[min(ib + q * kT + tid, n4 - 1)];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = ib + q * kT + tid;
        const float x[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * i + c;
          const uint32_t key = dense_key(t, i < n4, j, x[c]);
          f(j, key >= lo ? key : 0u);
        }
      }
    }
  } else if (t.vec) {
    const float4* r4 = reinterpret_cast<const float4*>(t.row);
    const int n4 = t.n / 4;
    constexpr int kU = 2;
    for (int ib = 0; ib < n4; ib += kU * kT) {
      float4 v[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = ib + q * kT + tid;
        v[q] = (i < n4) ? r4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = ib + q * kT + tid;
        const float x[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = 4 * i + c;
          const uint32_t key = (i < n4) ? tile_key(t, j, x[c]) : 0u;
          f(j, key >= lo ? key : 0u);
        }
      }
    }
  } else {
    for (int jb = 0; jb < t.n; jb += kT) {
      const int j = jb + tid;
      const uint32_t key = (j < t.n) ? tile_key(t, j, t.row[j]) : 0u;
      f(j, key >= lo ? key : 0u);
    }
  }
}

// The tile's columns with key >= lo (lo >= 1) appended to the survivors
// (skey, scol) from sh.n_surv on; those at or past cap are counted in
// sh.n_surv but not stored.  With kHist their top-12-bit histogram is added
// to sh.hist too.  The order of the survivors is unspecified.  All threads
// call.
template <bool kPacked, bool kHist>
__device__ __forceinline__ void collect_tile(const Tile& t, uint32_t lo, TileShared& sh, uint32_t* skey,
                                             int32_t* scol, int cap) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (!kPacked && t.vec && t.slot_map == nullptr) {
    // a batch of 4 * kDenseBatch columns per thread: one wavefront prefix
    // sum and one LDS atomic per batch place the thread's survivors
    const float4* r4 = reinterpret_cast<const float4*>(t.row);
    const int n4 = t.n / 4;
    constexpr int kU = kDenseBatch;
    for (int ib = 0; ib < n4; ib += kU * kT) {
      float4 v[kU];
#pragma unroll
      for (int q = 0; q < kU; ++q) v[q] = r4[min(ib + q * kT + tid, n4 - 1)];
      uint32_t key[4 * kU];
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < kU; ++q) {
        const int i = ib + q * kT + tid;
        const float x[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t k = dense_key(t, i < n4, 4 * i + e, x[e]);
          k = k >= lo ? k : 0u;
          key[4 * q + e] = k;
          c += k != 0u ? 1u : 0u;
          if (kHist && k != 0u) atomicAdd(&sh.hist[k >> 20], 1u);
        }
      }
      uint32_t incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
      }
      const uint32_t wtot = __shfl(incl, 63, 64);
      if (wtot == 0u) continue;                          // uniform over the wavefront
      uint32_t b = 0;
      if (lane == 0) b = atomicAdd(&sh.n_surv, wtot);
      uint32_t pos = __shfl(b, 0, 64) + incl - c;
#pragma unroll
      for (int e = 0; e < 4 * kU; ++e) {
        if (key[e] != 0u) {
          if (pos < static_cast<uint32_t>(cap)) {
            skey[pos] = key[e];
            scol[pos] = 4 * (ib + (e / 4) * kT + tid) + (e % 4);
          }
          ++pos;
        }
      }
    }
    return;
  }
  // one column per lane at a time: a ballot places the wavefront's survivors
  for_tile<kPacked, false>(t, lo, [&](int j, uint32_t key) {
    if (kHist && key != 0u) atomicAdd(&sh.hist[key >> 20], 1u);
    const bool s = key != 0u;
    const uint64_t m = __ballot(s);
    if (m == 0ull) return;
    uint32_t b = 0;
    if (lane == 0) b = atomicAdd(&sh.n_surv, static_cast<uint32_t>(__popcll(m)));
    b = __shfl(b, 0, 64);
    const uint32_t pos = b + static_cast<uint32_t>(__popcll(m & lanemask_lt(lane)));
    if (s && pos < static_cast<uint32_t>(cap)) {
      skey[pos] = key;
      scol[pos] = static_cast<int32_t>(j);
    }
  });
}

}  // namespace

// dyn LDS: ckey[k_total] | 8 * cap_lds bytes | bits[nw].  The running
// candidates' keys take ckey[0, c0); the survivors (key, column) take the
// rest up to bits, so a call with fewer running candidates (the first tile)
// holds more of them.  kPacked: the tile is in the packed form (p.tile_mask).
template <bool kPacked>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(8, 8))) void select_tile_kernel(
    SelectParams p, const float* scores, int cap_lds) {
  extern __shared__ uint32_t dyn[];
  __shared__ TileShared sh;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kcap = p.k_total;
  uint32_t* ckey = dyn;
  uint32_t* bits = dyn + kcap + 2 * cap_lds;
  const int nw = static_cast<int>((p.n + 31) / 32);

  Tile t;
  t.row = scores + static_cast<int64_t>(u) * p.row_stride;
  t.mask = p.tile_mask ? p.tile_mask + static_cast<int64_t>(u) * ((p.n + 63) / 64) : nullptr;
  t.n = static_cast<int>(p.n);
  t.base = static_cast<int>(p.base);
  t.sink_end = static_cast<int>(min(static_cast<int64_t>(p.n_sink), p.n_total));
  t.rec_begin = static_cast<int>(max(static_cast<int64_t>(t.sink_end), p.n_total - static_cast<int64_t>(p.n_recent)));
  t.slot_map = p.slot_map;
  t.dead = p.dead_slot;
  t.vec = (reinterpret_cast<uintptr_t>(t.row) & 15) == 0 && (p.n & 3) == 0;
  auto alive = [&](int64_t g) {
    return p.slot_map == nullptr || static_cast<int64_t>(p.slot_map[g]) != p.dead_slot;
  };

  // ---- alive forced entries of the whole unit, and the room left for the rest
  uint32_t fs = 0, fr = 0;
  for (int64_t g = tid; g < t.sink_end; g += kT) fs += alive(g) ? 1u : 0u;
  for (int64_t g = t.rec_begin + tid; g < p.n_total; g += kT) fr += alive(g) ? 1u : 0u;
  const uint32_t fsum = block_sum_u32(fs, sh);
  const uint32_t rsum = block_sum_u32(fr, sh);
  const int32_t room = p.k_total - static_cast<int32_t>(fsum + rsum);

  // ---- running candidates: keys to LDS (their indices are read at the end)
  const int c0 = min(max(p.cand_count[u], 0), max(room, 0));
  // survivors after the c0 keys: [c0, c0 + cap) keys, then cap columns,
  // ending at or before bits (c0 <= room <= k_total)
  const int cap = cap_lds + (kcap - c0) / 2;
  uint32_t* skey = ckey + c0;
  int32_t* scol = reinterpret_cast<int32_t*>(skey + cap);
  const int cpt = (c0 + kT - 1) / kT;                       // <= kMaxCandPerThread
  const int e0 = min(c0, tid * cpt), e1 = min(c0, e0 + cpt);
  const int64_t cbase = static_cast<int64_t>(u) * kcap;
  for (int e = e0; e < e1; ++e) ckey[e] = score_key(p.cand_score[cbase + e]);
  for (int b = tid; b < kBins; b += kT) sh.hist[b] = 0u;
  if (tid == 0) sh.n_surv = 0u;
  __syncthreads();
  uint32_t mk = 0xFFFFFFFFu;
  for (int e = e0; e < e1; ++e) mk = min(mk, ckey[e]);
  const uint32_t cmin = block_min_u32(mk, sh);
  // a full running set makes its smallest key a threshold for the tile
  const uint32_t lo0 = (room > 0 && c0 == room) ? cmin + 1u : 1u;

  // ---- pass 1: survivors (key >= lo0) to LDS and the top-12-bit histogram
  uint32_t lo = lo0;
  for (int e = e0; e < e1; ++e) atomicAdd(&sh.hist[ckey[e] >> 20], 1u);
  if (room > 0) collect_tile<kPacked, true>(t, lo, sh, skey, scol, cap);
  __syncthreads();
  uint32_t n_tile = sh.n_surv;                    // tile entries >= lo (may exceed cap)
  bool in_lds = n_tile <= static_cast<uint32_t>(cap);
  const uint32_t n_all = static_cast<uint32_t>(c0) + n_tile;
  // the admission threshold when every entry is taken and exactly fills the
  // set: the smallest of them (survivors read back from LDS; 0 = none known)
  uint32_t full_min = 0u;
  if (!p.finalize && p.admit != nullptr && room > 0 && n_all == static_cast<uint32_t>(room) && in_lds) {
    uint32_t m = 0xFFFFFFFFu;
    for (uint32_t i = tid; i < n_tile; i += kT) m = min(m, skey[i]);
    full_min = min(cmin, block_min_u32(m, sh));
  }

  // ---- radix select of the room-th largest key over candidates + tile
  uint32_t T;
  int32_t remaining;
  if (room <= 0) {
    T = 0xFFFFFFFFu;                              // no finite score maps here: nothing selected
    remaining = 0;
  } else if (n_all <= static_cast<uint32_t>(room)) {
    T = 1u;                                       // every entry is above
    remaining = 0;
  } else {
    uint32_t prefix = 0u, rem = static_cast<uint32_t>(room), n_above = 0u;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int d = 0; d < 3; ++d) {
      const int sh_d = shifts[d];
      const uint32_t hi_mask = (d == 0) ? 0u : (0xFFFFFFFFu << (sh_d + widths[d]));
      const uint32_t dmask = (1u << widths[d]) - 1u;
      if (d > 0) {
        for (int b = tid; b < kBins; b += kT) sh.hist[b] = 0u;
        __syncthreads();
        for (int e = e0; e < e1; ++e) {
          const uint32_t key = ckey[e];
          if (((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> sh_d) & dmask], 1u);
        }
        if (in_lds) {
          for (uint32_t s = tid; s < n_tile; s += kT) {
            const uint32_t key = skey[s];
            if (((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> sh_d) & dmask], 1u);
          }
        } else {
          for_tile<kPacked>(t, lo, [&](int, uint32_t key) {
            if (key != 0u && ((key ^ prefix) & hi_mask) == 0u) atomicAdd(&sh.hist[(key >> sh_d) & dmask], 1u);
          });
        }
        __syncthreads();
      }
      find_bin_block(sh, 1 << widths[d], rem);
      prefix |= sh.bin << sh_d;
      n_above += sh.above;
      rem = sh.rem;
      const uint32_t in_bin = sh.hist[sh.bin];
      __syncthreads();
      if (!in_lds && d < 2 && n_above + in_bin <= static_cast<uint32_t>(cap)) {
        // the entries at or above this bin fit: read the tile once more and keep only those
        lo = max(lo0, prefix);
        if (tid == 0) sh.n_surv = 0u;
        __syncthreads();
        collect_tile<kPacked, false>(t, lo, sh, skey, scol, cap);
        __syncthreads();
        n_tile = sh.n_surv;
        in_lds = true;                            // n_tile <= n_above + in_bin <= cap
      }
    }
    T = prefix;
    remaining = static_cast<int32_t>(rem);
  }

  // The admission threshold for the next tile (nothing in this launch reads
  // it): the new running set's smallest key once the set is full -- T when
  // the radix select ran (room entries with keys >= T are taken, at least
  // one equal to T), full_min when every entry is taken and fills it; a
  // later column enters only above it.  NaN (admit everything) otherwise.
  if (tid == 0 && !p.finalize && p.admit != nullptr) {
    uint32_t thr = 0u;
    if (room > 0 && n_all > static_cast<uint32_t>(room)) thr = T;
    else if (room > 0 && n_all == static_cast<uint32_t>(room)) thr = full_min;
    p.admit[u] = thr != 0u ? key_score(thr) : __uint_as_float(0x7FC00000u);
  }

  // ---- candidates: ranks among keys equal to T, then positions (array order)
  uint32_t my_eq = 0;
  for (int e = e0; e < e1; ++e) my_eq += (ckey[e] == T) ? 1u : 0u;
  uint32_t eq_c;
  const uint32_t eq_before = block_exclusive(my_eq, sh, &eq_c);
  const uint32_t take_c_eq = min(eq_c, static_cast<uint32_t>(max(remaining, 0)));
  const uint32_t take_t_eq = static_cast<uint32_t>(max(remaining, 0)) - take_c_eq;
  uint32_t csel_mask = 0u, my_sel = 0u;
  {
    uint32_t r = eq_before;
#pragma unroll
    for (int i = 0; i < kMaxCandPerThread; ++i) {
      const int e = e0 + i;
      if (e < e1) {
        const uint32_t key = ckey[e];
        bool sel = key > T;
        if (key == T) {
          sel = r < take_c_eq;
          ++r;
        }
        if (sel) {
          csel_mask |= 1u << i;
          ++my_sel;
        }
      }
    }
  }
  uint32_t n_sel_c;
  const uint32_t csel_before = block_exclusive(my_sel, sh, &n_sel_c);

  // ---- tile entries: equal-to-T ranks by column, when only some are taken
  auto visit = [&](auto&& f) {
    if (in_lds) {
      for (uint32_t s = tid; s < n_tile; s += kT) f(scol[s], skey[s]);
    } else {
      for_tile<kPacked, false>(t, lo, [&](int j, uint32_t key) {
        if (key != 0u) f(j, key);
      });
    }
  };
  auto clear_bits = [&]() {
    for (int w = tid; w < nw; w += kT) bits[w] = 0u;
  };
  // per-thread exclusive prefix of the set bits; thread tid owns words [tid*wpt, ...)
  const int wpt = (nw + kT - 1) / kT;
  auto scan_bits = [&]() {
    const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
    uint32_t c = 0;
    for (int w = w0; w < w1; ++w) c += __popc(bits[w]);
    uint32_t tot;
    const uint32_t ex = block_exclusive(c, sh, &tot);
    sh.scan[tid] = ex;
    __syncthreads();
    return tot;
  };
  auto rank_of = [&](int j) {
    const int w = j >> 5;
    const int owner = w / wpt;
    uint32_t r = sh.scan[owner];
    for (int x = owner * wpt; x < w; ++x) r += __popc(bits[x]);
    return r + static_cast<uint32_t>(__popc(bits[w] & ((1u << (j & 31)) - 1u)));
  };

  // equal-to-T tile columns are taken in ascending column order up to
  // take_t_eq: find the column of the last one taken (cstar) when only some are
  uint32_t eq_t = 0;
  {
    uint32_t c = 0;
    if (take_t_eq > 0) visit([&](int, uint32_t key) { c += (key == T) ? 1u : 0u; });
    eq_t = block_sum_u32(c, sh);
  }
  const bool rank_eq = take_t_eq > 0 && take_t_eq < eq_t;
  int cstar = t.n;                                // every equal-to-T column is taken
  if (rank_eq) {
    clear_bits();
    __syncthreads();
    visit([&](int j, uint32_t key) {
      if (key == T) atomicOr(&bits[j >> 5], 1u << (j & 31));
    });
    __syncthreads();
    scan_bits();
    // the thread whose words hold the bit of rank take_t_eq - 1 finds its column
    const int w0 = min(nw, tid * wpt), w1 = min(nw, w0 + wpt);
    uint32_t r = sh.scan[tid];
    for (int w = w0; w < w1; ++w) {
      uint32_t b = bits[w];
      const uint32_t c = __popc(b);
      if (r <= take_t_eq - 1 && take_t_eq - 1 < r + c) {
        for (uint32_t skip = take_t_eq - 1 - r; skip > 0; --skip) b &= b - 1;
        sh.bin = static_cast<uint32_t>(w * 32 + (__ffs(b) - 1));
      }
      r += c;
    }
    __syncthreads();
    cstar = static_cast<int>(sh.bin);
    __syncthreads();
  }
  // selected tile columns: key > T, or equal to T at a column <= cstar
  auto tile_selected = [&](int j, uint32_t key) {
    return key > T || (key == T && take_t_eq > 0 && j <= cstar);
  };
  clear_bits();
  __syncthreads();
  visit([&](int j, uint32_t key) {
    if (key != 0u && tile_selected(j, key)) atomicOr(&bits[j >> 5], 1u << (j & 31));
  });
  __syncthreads();
  const uint32_t n_sel_t = scan_bits();
  const uint32_t n_sel = n_sel_c + n_sel_t;

  // ---- outputs in ascending global index: selected candidates, then tile columns.
  // The candidates' indices are read before the barrier: a non-final call
  // writes its output over the same buffer.
  int32_t cidx[kMaxCandPerThread];
#pragma unroll
  for (int i = 0; i < kMaxCandPerThread; ++i) {
    const int e = e0 + i;
    cidx[i] = (e < e1 && (csel_mask & (1u << i))) ? p.cand_idx[cbase + e] : -1;
  }
  __syncthreads();
  const bool fin = p.finalize != 0;
  int32_t* kept = p.kept_idx + static_cast<int64_t>(u) * p.k_total;
  const uint32_t out0 = fin ? fsum : 0u;
  {
    uint32_t r = csel_before;
#pragma unroll
    for (int i = 0; i < kMaxCandPerThread; ++i) {
      const int e = e0 + i;
      if (e < e1 && (csel_mask & (1u << i))) {
        if (fin) {
          kept[out0 + r] = cidx[i];
        } else {
          p.cand_score[cbase + r] = key_score(ckey[e]);
          p.cand_idx[cbase + r] = cidx[i];
        }
        ++r;
      }
    }
  }
  visit([&](int j, uint32_t key) {
    if (key == 0u || !(bits[j >> 5] & (1u << (j & 31)))) return;
    const uint32_t r = n_sel_c + rank_of(j);
    const int32_t g = t.base + j;
    if (fin) {
      kept[out0 + r] = g;
    } else {
      p.cand_score[cbase + r] = key_score(key);
      p.cand_idx[cbase + r] = g;
    }
  });
  if (!fin) {
    if (tid == 0) {
      p.cand_count[u] = static_cast<int32_t>(n_sel);
    }
    return;
  }
  // ---- forced entries: alive sink first, alive recent last
  const int wave = tid >> 6;
  if (wave == 0) {
    uint32_t r = 0;
    for (int64_t g0 = 0; g0 < t.sink_end; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < t.sink_end && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  } else if (wave == 1) {
    uint32_t r = fsum + n_sel;
    for (int64_t g0 = t.rec_begin; g0 < p.n_total; g0 += 64) {
      const int64_t g = g0 + lane;
      const bool a = g < p.n_total && alive(g);
      const uint64_t b = __ballot(a);
      if (a) kept[r + __popcll(b & lanemask_lt(lane))] = static_cast<int32_t>(g);
      r += __popcll(b);
    }
  }
  const int64_t total = static_cast<int64_t>(fsum) + n_sel + rsum;
  for (int64_t i = total + tid; i < p.k_total; i += kT) kept[i] = -1;
  if (tid == 0 && p.n_kept != nullptr) p.n_kept[u] = static_cast<int32_t>(total);
}

}  // namespace kvsel

namespace kvsel {

namespace {
constexpr int64_t kLdsBytes = 160 * 1024;

// Survivor capacity for a tile call, or 0 if the call does not fit in LDS
// (the caller then takes the general two-launch path).  Two workgroups per
// compute unit when the survivors still hold one running set plus a margin,
// else one.
int tile_cap(const SelectParams& p, size_t* dyn_bytes) {
  const int64_t fixed = static_cast<int64_t>(sizeof(TileShared)) + 4 * (p.k_total + (p.n + 31) / 32);
  int64_t cap = (kLdsBytes / 2 - fixed) / 8;
  if (cap < static_cast<int64_t>(p.k_total) + 256) cap = (kLdsBytes - fixed) / 8;
  if (cap < 256) return 0;
  cap = min(cap, static_cast<int64_t>(1) << 20);
  *dyn_bytes = static_cast<size_t>(fixed - static_cast<int64_t>(sizeof(TileShared)) + 8 * cap);
  return static_cast<int>(cap);
}
}  // namespace

bool select_tile_fits(const SelectParams& p) {
  size_t dyn = 0;
  return p.cand_count != nullptr && p.k_total <= kMaxCandPerThread * kT && tile_cap(p, &dyn) > 0;
}

hipError_t launch_select_tile(const SelectParams& p, const float* scores, hipStream_t st) {
  size_t dyn = 0;
  const int cap = tile_cap(p, &dyn);
  const void* kern = p.tile_mask != nullptr ? reinterpret_cast<const void*>(&select_tile_kernel<true>)
                                             : reinterpret_cast<const void*>(&select_tile_kernel<false>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(dyn));
  if (e != hipSuccess) return e;
  if (p.tile_mask != nullptr) select_tile_kernel<true><<<p.U, kT, dyn, st>>>(p, scores, cap);
  else select_tile_kernel<false><<<p.U, kT, dyn, st>>>(p, scores, cap);
  return hipGetLastError();
}

}  // namespace kvsel
