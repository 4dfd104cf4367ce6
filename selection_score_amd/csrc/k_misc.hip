// Slot-map redirect, dead-slot sentinel rows, and the session memory update.
#include "common.h"

#include <math.h>

namespace kvsel {

// IntentKV §4 (redirect): dropped positions point at the dead slot; kept
// positions keep their slot ids.
__global__ void redirect_kernel(int64_t N, int32_t* __restrict__ slot_map,
                                const uint8_t* __restrict__ keep, int32_t dead) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j < N && keep[j] == 0) slot_map[j] = dead;
}

// The same with the kept positions as an ascending list (kvsel_select's
// kept_idx, -1 past its count): j is kept iff it is in the list, found by a
// binary search where negative entries sort last.
__global__ void redirect_list_kernel(int64_t N, int32_t* __restrict__ slot_map,
                                     const int32_t* __restrict__ kept, int32_t k, int32_t dead) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= N) return;
  int lo = 0, hi = k - 1;
  bool found = false;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int64_t v = kept[mid] < 0 ? INT64_MAX : static_cast<int64_t>(kept[mid]);
    if (v == j) {
      found = true;
      break;
    }
    if (v < j) lo = mid + 1;
    else hi = mid - 1;
  }
  if (!found) slot_map[j] = dead;
}

// IntentKV §2 Q2: the dead slot holds K = -1e4 (rounded to the pool's
// 16-bit format) and V = 0 in every layer and KV head.
__global__ void sentinel_kernel(uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                                int L, int Hkv, int D, uint16_t k_bits, int64_t pool_slots,
                                int64_t dead) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_layer = static_cast<int64_t>(Hkv) * D;
  if (i >= per_layer * L) return;
  const int64_t l = i / per_layer, r = i % per_layer;
  const int64_t off = (l * pool_slots + dead) * per_layer + r;
  k_pool[off] = k_bits;
  v_pool[off] = 0;
}

// IntentKV §4 (memory recurrence) and §7 (unit-norm projection): one
// wavefront per (layer, query head).
template <int DT>
__global__ __launch_bounds__(256) void memory_update_kernel(int LH, int D, int W,
                                                            const void* __restrict__ q,
                                                            float* __restrict__ M, float decay) {
  const int lane = threadIdx.x & 63;
  const int lh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (lh >= LH) return;
  float m[4];
  float nn = 0.f;
  for (int c = 0; c < 4; ++c) {
    const int d = lane + 64 * c;
    m[c] = 0.f;
    if (d >= D) continue;
    float s = 0.f;
    for (int t = 0; t < W; ++t) s += load_elem<DT>(q, (static_cast<int64_t>(lh) * W + t) * D + d);
    m[c] = decay * M[static_cast<int64_t>(lh) * D + d] + s / static_cast<float>(W);
    nn += m[c] * m[c];
  }
  for (int o = 32; o > 0; o >>= 1) nn += __shfl_xor(nn, o, 64);
  const float inv = (nn > 0.f) ? 1.0f / sqrtf(nn) : 0.f;
  for (int c = 0; c < 4; ++c) {
    const int d = lane + 64 * c;
    if (d < D) M[static_cast<int64_t>(lh) * D + d] = m[c] * inv;
  }
}

// The same update with 16-byte loads: lane (row group rs, column piece rl)
// sums its piece over rows rs, rs + 64 / lpr, ... with eight loads in flight;
// the row groups are then summed across lanes.  Needs D * esz in
// {128, 256, 512, 1024} and 16-byte aligned query rows.
template <int DT>
__global__ __launch_bounds__(256) void memory_update_vec_kernel(int LH, int D, int W,
                                                                const void* __restrict__ q,
                                                                float* __restrict__ M, float decay) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = 16 / esz;
  constexpr int kRowBatch = 8;
  const int lane = threadIdx.x & 63;
  const int lh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (lh >= LH) return;                           // the whole wavefront
  const int lpr = D * esz / 16;                   // 8, 16, 32 or 64 lanes per row
  const int rpp = 64 / lpr;                       // rows per pass
  const int rl = lane % lpr, rs = lane / lpr;
  const int64_t row_bytes = static_cast<int64_t>(D) * esz;
  const uint8_t* base = static_cast<const uint8_t*>(q) + static_cast<int64_t>(lh) * W * row_bytes + rl * 16;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int t0 = rs; t0 < W; t0 += rpp * kRowBatch) {
    uint4 v[kRowBatch];
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      const int t = t0 + j * rpp;
      v[j] = (t < W) ? *reinterpret_cast<const uint4*>(base + t * row_bytes) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kRowBatch; ++j) {
      if (t0 + j * rpp >= W) break;
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      if constexpr (DT == KVSEL_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(w[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t lo = static_cast<uint16_t>(w[i] & 0xFFFFu), hi = static_cast<uint16_t>(w[i] >> 16);
          acc[2 * i] += (DT == KVSEL_BF16) ? bf16_to_f32(lo) : f16_to_f32(lo);
          acc[2 * i + 1] += (DT == KVSEL_BF16) ? bf16_to_f32(hi) : f16_to_f32(hi);
        }
      }
    }
  }
  for (int o = lpr; o < 64; o <<= 1)              // every lane of a column piece ends with its total
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  float m[E];
  float nn = 0.f;
  float* mrow = M + static_cast<int64_t>(lh) * D + rl * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    m[e] = decay * mrow[e] + acc[e] / static_cast<float>(W);
    nn += m[e] * m[e];
  }
  for (int o = 1; o < lpr; o <<= 1) nn += __shfl_xor(nn, o, 64);
  const float inv = (nn > 0.f) ? 1.0f / sqrtf(nn) : 0.f;
  if (rs == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) mrow[e] = m[e] * inv;
  }
}

// ---- alias-aware free list (IntentKV §7): bitmaps over the slot ids of the
// kept positions and of the dropped ones, then one workgroup lists the slots
// that are dropped and not kept in ascending order.
__global__ void free_clear_kernel(uint32_t* bits, int64_t n_words) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n_words) bits[i] = 0u;
}

// kept_bits: slots of kept positions; drop_bits: slots of dropped positions
// outside the protected prefix, other than the dead slot.  A slot is freed
// when it is in drop_bits and not in kept_bits.
// Lanes whose slots share a bitmap word are merged into one atomicOr: the
// leading active lane's word is OR-reduced over the wavefront, up to
// kOrRounds distinct words; lanes left after that add their bit alone.
// Every lane of the wavefront must take part.
constexpr int kOrRounds = 8;
__device__ __forceinline__ void wave_or_bit(uint32_t* bits, int64_t word, uint32_t bit, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t left = __ballot(active);
  for (int round = 0; round < kOrRounds && left != 0ull; ++round) {
    const int leader = __ffsll(static_cast<long long>(left)) - 1;
    const int64_t w = __shfl(word, leader, 64);
    const bool mine = active && word == w;
    uint32_t m = mine ? bit : 0u;
    for (int o = 1; o < 64; o <<= 1) m |= __shfl_xor(m, o, 64);
    if (lane == leader) atomicOr(&bits[w], m);
    left &= ~__ballot(mine);
    if (mine) active = false;
  }
  if (active) atomicOr(&bits[word], bit);
}

__global__ __launch_bounds__(256) void free_mark_kernel(int64_t N, const int32_t* __restrict__ slot_map,
                                                        const uint8_t* __restrict__ keep, int64_t dead,
                                                        int64_t protected_len, int64_t n_slots,
                                                        uint32_t* __restrict__ kept_bits,
                                                        uint32_t* __restrict__ drop_bits) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool in = j < N;                            // every lane stays for the wavefront-wide merges
  const int64_t u = in ? slot_map[j] : -1;
  const bool valid = in && u >= 0 && u < n_slots;
  const bool kept = valid && keep[j] != 0;
  const bool dropped = valid && !kept && j >= protected_len && u != dead;
  const uint32_t bit = 1u << (u & 31);
  wave_or_bit(kept_bits, u >> 5, bit, kept);
  wave_or_bit(drop_bits, u >> 5, bit, dropped);
}

// One workgroup: wavefront w owns a contiguous run of bitmap words.  The
// wavefronts' counts give each run its first output index; each wavefront
// then walks its words two at a time (lane l looks at bit l % 32 of word
// l / 32) and stores the set bits' slot ids with a ballot prefix, so every
// store instruction writes consecutive outputs.
constexpr int kFreeThreads = 1024;
constexpr int kFreeWaves = kFreeThreads / 64;
__global__ __launch_bounds__(kFreeThreads) void free_compact_kernel(int64_t N, int64_t n_words,
                                                                    const uint32_t* __restrict__ kept_bits,
                                                                    const uint32_t* __restrict__ drop_bits,
                                                                    int32_t* __restrict__ free_slots,
                                                                    int32_t* __restrict__ n_free) {
  __shared__ uint32_t wave_tot[kFreeWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = (n_words + kFreeWaves - 1) / kFreeWaves;
  const int64_t w0 = min(n_words, static_cast<int64_t>(wave) * per);
  const int64_t w1 = min(n_words, w0 + per);
  uint32_t cnt = 0;
  for (int64_t w = w0 + lane; w < w1; w += 64) cnt += __popc(drop_bits[w] & ~kept_bits[w]);
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) wave_tot[wave] = cnt;
  __syncthreads();
  uint32_t base = 0, total = 0;
  for (int w = 0; w < kFreeWaves; ++w) {
    if (w < wave) base += wave_tot[w];
    total += wave_tot[w];
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = w0; c0 < w1; c0 += 64) {
    // 64 words in registers (one per lane), handed out two per step
    const int64_t mine = c0 + lane;
    const uint32_t word = (mine < w1) ? (drop_bits[mine] & ~kept_bits[mine]) : 0u;
    const int steps = static_cast<int>((min(w1 - c0, static_cast<int64_t>(64)) + 1) / 2);
    for (int t = 0; t < steps; ++t) {
      const int src = 2 * t + (lane >> 5);
      const uint32_t wv = __shfl(word, src, 64);            // word c0 + src (0 past w1)
      const bool set = ((wv >> (lane & 31)) & 1u) != 0u;
      const uint64_t b = __ballot(set);
      if (set) free_slots[base + __popcll(b & lt)] = static_cast<int32_t>((c0 + src) * 32 + (lane & 31));
      base += static_cast<uint32_t>(__popcll(b));
    }
  }
  for (int64_t i = static_cast<int64_t>(total) + tid; i < N; i += kFreeThreads) free_slots[i] = -1;
  if (tid == 0) n_free[0] = static_cast<int32_t>(total);
}

size_t free_list_workspace_bytes(int64_t n_slots) {
  const int64_t words = (n_slots + 31) / 32;
  return static_cast<size_t>(2 * ((words * 4 + 255) / 256 * 256));
}

hipError_t launch_free_list(int64_t N, const int32_t* slot_map, const uint8_t* keep, int64_t dead,
                            int64_t protected_len, int64_t n_slots, int32_t* free_slots, int32_t* n_free,
                            void* ws, hipStream_t st) {
  const int64_t words = (n_slots + 31) / 32;
  uint32_t* kept_bits = static_cast<uint32_t*>(ws);
  uint32_t* drop_bits = kept_bits + (words * 4 + 255) / 256 * 64;
  const int64_t all_words = (drop_bits - kept_bits) + words;   // both bitmaps, one clear
  free_clear_kernel<<<static_cast<int>(ceil_div(all_words, 256)), 256, 0, st>>>(kept_bits, all_words);
  if (N > 0) {
    free_mark_kernel<<<static_cast<int>(ceil_div(N, 256)), 256, 0, st>>>(N, slot_map, keep, dead, protected_len,
                                                                        n_slots, kept_bits, drop_bits);
  }
  free_compact_kernel<<<1, kFreeThreads, 0, st>>>(N, words, kept_bits, drop_bits, free_slots, n_free);
  return hipGetLastError();
}

hipError_t launch_redirect(int64_t N, int32_t* slot_map, const uint8_t* keep, int64_t dead,
                           hipStream_t st) {
  if (N == 0) return hipSuccess;
  redirect_kernel<<<static_cast<int>(ceil_div(N, 256)), 256, 0, st>>>(N, slot_map, keep,
                                                                     static_cast<int32_t>(dead));
  return hipGetLastError();
}

hipError_t launch_redirect_list(int64_t N, int32_t* slot_map, const int32_t* kept_idx, int32_t k, int64_t dead,
                                hipStream_t st) {
  if (N == 0) return hipSuccess;
  redirect_list_kernel<<<static_cast<int>(ceil_div(N, 256)), 256, 0, st>>>(N, slot_map, kept_idx, k,
                                                                          static_cast<int32_t>(dead));
  return hipGetLastError();
}

hipError_t launch_sentinel(void* k_pool, void* v_pool, int L, int Hkv, int D, int dtype,
                           int64_t pool_slots, int64_t dead, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(L) * Hkv * D;
  if (n == 0) return hipSuccess;
  // -1e4 rounded to the storage format: bf16 -9984 (0xC61C), f16 -10000 (0xF0E2)
  const uint16_t bits = (dtype == KVSEL_BF16) ? 0xC61Cu : 0xF0E2u;
  sentinel_kernel<<<static_cast<int>(ceil_div(n, 256)), 256, 0, st>>>(
      static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), L, Hkv, D, bits, pool_slots,
      dead);
  return hipGetLastError();
}

hipError_t launch_memory_update(int L, int Hq, int D, int W, int dt, const void* q, float* M,
                                float decay, hipStream_t st) {
  const int LH = L * Hq;
  if (LH == 0) return hipSuccess;
  const int grid = static_cast<int>(ceil_div(LH, 4));
  const int esz = (dt == KVSEL_F32) ? 4 : 2;
  const int row = D * esz;
  if ((row == 128 || row == 256 || row == 512 || row == 1024) && (reinterpret_cast<uintptr_t>(q) & 15) == 0) {
    if (dt == KVSEL_BF16) memory_update_vec_kernel<KVSEL_BF16><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
    else if (dt == KVSEL_F16) memory_update_vec_kernel<KVSEL_F16><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
    else memory_update_vec_kernel<KVSEL_F32><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
    return hipGetLastError();
  }
  if (dt == KVSEL_BF16) memory_update_kernel<KVSEL_BF16><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
  else if (dt == KVSEL_F16) memory_update_kernel<KVSEL_F16><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
  else memory_update_kernel<KVSEL_F32><<<grid, 256, 0, st>>>(LH, D, W, q, M, decay);
  return hipGetLastError();
}

}  // namespace kvsel
