// Mean-K index build.
//
// KVMem (query-conditioned retrieval paragraph): the block scorer reads one
// RoPE-stripped mean key per (layer, KV head, 32-token block), kept in HBM as
// an fp16 index that grows as blocks fill.  A wavefront takes 64 / (D * esz
// / 16) consecutive blocks at a time (4 for bf16 rows of 128): each lane owns
// one 16-byte column piece of one block and sums that piece over all the
// block's rows in float64, eight rows in flight at a time, so no cross-lane
// reduction is needed.  The float64 sum is exact for a block's 32 bf16 or
// f16 rows (and for float32 rows spanning fewer than 2^29 in magnitude); it
// is divided by the block size in float64 and rounded once to fp16.
#include "common.h"

namespace kvsel {

namespace {

typedef unsigned int ix_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kIndexBatch = 8;        // 16-byte row pieces per lane in flight

// float64 -> fp16 bits with a single round to nearest even.  The value is
// first narrowed to float32 by truncation with the last bit forced to 1 when
// anything was cut off (round-to-odd); float32 keeps more than two bits
// beyond fp16's, so the final RNE step to fp16 rounds as the float64 value
// itself would.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  float t = __double2float_rz(x);
  if (static_cast<double>(t) != x) t = __uint_as_float(__float_as_uint(t) | 1u);
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(t));
}

template <int DT>
__device__ __forceinline__ void add_piece(double* acc, const ix_u32x4& v) {
  if constexpr (DT == KVSEL_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += static_cast<double>(__uint_as_float(v[e]));
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = v[w] & 0xFFFFu, hi = v[w] >> 16;
      float a, b;
      if constexpr (DT == KVSEL_BF16) {
        a = __uint_as_float(lo << 16);
        b = __uint_as_float(hi << 16);
      } else {
        a = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(lo)));
        b = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hi)));
      }
      acc[2 * w] += static_cast<double>(a);
      acc[2 * w + 1] += static_cast<double>(b);
    }
  }
}

}  // namespace

template <int DT>
__global__ __launch_bounds__(256) void mean_k_kernel(IndexParams p, const void* __restrict__ src,
                                                     uint16_t* __restrict__ mu) {
  constexpr int esz = (DT == KVSEL_F32) ? 4 : 2;
  constexpr int E = 16 / esz;                     // elements per 16-byte piece
  const int lane = threadIdx.x & 63;
  const int lpr = p.D * esz / 16;                 // lanes per row: 8, 16 or 32
  const int bpw = 64 / lpr;                       // blocks per wavefront at a time: 8, 4 or 2
  const int rlane = lane % lpr, slot = lane / lpr;
  const int64_t row_bytes = static_cast<int64_t>(p.D) * esz;
  const int64_t items = static_cast<int64_t>(p.U) * p.b_count;
  const int64_t wave_global = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / 64;
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * blockDim.x / 64;
  const double count = static_cast<double>(p.bt);
  for (int64_t it0 = wave_global * bpw; it0 < items; it0 += n_waves * bpw) {
    const int64_t it = it0 + slot;
    const bool live = it < items;
    const int64_t itc = live ? it : items - 1;
    const int u = static_cast<int>(itc / p.b_count);
    const int64_t b = p.b_begin + (itc - static_cast<int64_t>(u) * p.b_count);
    const int64_t off = p.src_offsets ? p.src_offsets[u] : static_cast<int64_t>(u) * p.src_unit_stride;
    const uint8_t* blk = static_cast<const uint8_t*>(src) + off * esz + b * p.bt * row_bytes + rlane * 16;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;       // the sum starts from 0: a block of -0 rows gives +0
    for (int r0 = 0; r0 < p.bt; r0 += kIndexBatch) {
      ix_u32x4 v[kIndexBatch];
#pragma unroll
      for (int j = 0; j < kIndexBatch; ++j)
        v[j] = (r0 + j < p.bt) ? *reinterpret_cast<const ix_u32x4*>(blk + (r0 + j) * row_bytes)
                               : ix_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kIndexBatch; ++j)
        if (r0 + j < p.bt) add_piece<DT>(acc, v[j]);
    }
    if (live) {
      uint16_t h[E];
#pragma unroll
      for (int e = 0; e < E; ++e) h[e] = f64_to_f16_bits(acc[e] / count);   // IEEE float64 division
      uint16_t* dst = mu + ((static_cast<int64_t>(u) * p.NB + b) * p.D + rlane * E);
      if constexpr (E == 8) {
        uint4 w;
        w.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
        w.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
        w.z = h[4] | (static_cast<uint32_t>(h[5]) << 16);
        w.w = h[6] | (static_cast<uint32_t>(h[7]) << 16);
        store16_stream(dst, w);
      } else {
        uint2 w;
        w.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
        w.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
        *reinterpret_cast<uint2*>(dst) = w;
      }
    }
  }
}

hipError_t launch_build_index(const IndexParams& p, const void* src_k, uint16_t* mu, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(p.U) * p.b_count;
  if (items == 0) return hipSuccess;
  const int64_t blocks = ceil_div(items, 4 * 4);   // a few blocks per wavefront at a time
  const int grid = static_cast<int>(blocks > 65536 ? 65536 : blocks);
  if (p.dtype == KVSEL_BF16) mean_k_kernel<KVSEL_BF16><<<grid, 256, 0, st>>>(p, src_k, mu);
  else if (p.dtype == KVSEL_F16) mean_k_kernel<KVSEL_F16><<<grid, 256, 0, st>>>(p, src_k, mu);
  else mean_k_kernel<KVSEL_F32><<<grid, 256, 0, st>>>(p, src_k, mu);
  return hipGetLastError();
}

}  // namespace kvsel
