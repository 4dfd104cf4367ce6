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
// kept positions and of the freeable ones, then one workgroup lists the set
// bits in ascending order.
__global__ void free_clear_kernel(uint32_t* bits, int64_t n_words) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n_words) bits[i] = 0u;
}

__global__ void free_mark_kept_kernel(int64_t N, const int32_t* __restrict__ slot_map,
                                      const uint8_t* __restrict__ keep, int64_t n_slots,
                                      uint32_t* __restrict__ kept_bits) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= N || keep[j] == 0) return;
  const int64_t u = slot_map[j];
  if (u >= 0 && u < n_slots) atomicOr(&kept_bits[u >> 5], 1u << (u & 31));
}

__global__ void free_mark_kernel(int64_t N, const int32_t* __restrict__ slot_map,
                                 const uint8_t* __restrict__ keep, int64_t dead, int64_t protected_len,
                                 int64_t n_slots, const uint32_t* __restrict__ kept_bits,
                                 uint32_t* __restrict__ free_bits) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= N || j < protected_len || keep[j] != 0) return;
  const int64_t u = slot_map[j];
  if (u == dead || u < 0 || u >= n_slots) return;
  const uint32_t bit = 1u << (u & 31);
  if ((kept_bits[u >> 5] & bit) == 0u) atomicOr(&free_bits[u >> 5], bit);
}

// One workgroup: thread t owns a contiguous run of bitmap words, so the
// exclusive scan of the per-thread counts gives every set bit its place.
constexpr int kFreeThreads = 1024;
__global__ __launch_bounds__(kFreeThreads) void free_compact_kernel(int64_t N, int64_t n_words,
                                                                    const uint32_t* __restrict__ free_bits,
                                                                    int32_t* __restrict__ free_slots,
                                                                    int32_t* __restrict__ n_free) {
  __shared__ uint32_t wave_tot[kFreeThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per = (n_words + kFreeThreads - 1) / kFreeThreads;
  const int64_t w0 = min(n_words, static_cast<int64_t>(tid) * per);
  const int64_t w1 = min(n_words, w0 + per);
  uint32_t cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(free_bits[w]);
  // exclusive scan over the workgroup: within the wavefront, then across
  uint32_t incl = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t base = incl - cnt, total = 0;
  for (int w = 0; w < kFreeThreads / 64; ++w) {
    if (w < wave) base += wave_tot[w];
    total += wave_tot[w];
  }
  uint32_t pos = base;
  for (int64_t w = w0; w < w1; ++w) {
    uint32_t b = free_bits[w];
    while (b != 0u) {
      const int i = __ffs(b) - 1;
      free_slots[pos++] = static_cast<int32_t>(w * 32 + i);
      b &= b - 1u;
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
  uint32_t* free_bits = kept_bits + (words * 4 + 255) / 256 * 64;
  const int64_t all_words = (free_bits - kept_bits) + words;   // both bitmaps, one clear
  free_clear_kernel<<<static_cast<int>(ceil_div(all_words, 256)), 256, 0, st>>>(kept_bits, all_words);
  if (N > 0) {
    const int g = static_cast<int>(ceil_div(N, 256));
    free_mark_kept_kernel<<<g, 256, 0, st>>>(N, slot_map, keep, n_slots, kept_bits);
    free_mark_kernel<<<g, 256, 0, st>>>(N, slot_map, keep, dead, protected_len, n_slots, kept_bits, free_bits);
  }
  free_compact_kernel<<<1, kFreeThreads, 0, st>>>(N, words, free_bits, free_slots, n_free);
  return hipGetLastError();
}

hipError_t launch_redirect(int64_t N, int32_t* slot_map, const uint8_t* keep, int64_t dead,
                           hipStream_t st) {
  if (N == 0) return hipSuccess;
  redirect_kernel<<<static_cast<int>(ceil_div(N, 256)), 256, 0, st>>>(N, slot_map, keep,
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
