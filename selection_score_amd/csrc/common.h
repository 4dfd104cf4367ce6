// Internal helpers shared by the libkvsel translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

// ---------------------------------------------------------------- element access

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 v = static_cast<_Float16>(f);
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

// Load element i of a buffer of the given storage type as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (DT == KVSEL_F32) {
    return static_cast<const float*>(p)[i];
  } else if constexpr (DT == KVSEL_BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return f16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
  if constexpr (DT == KVSEL_F32) {
    static_cast<float*>(p)[i] = v;
  } else if constexpr (DT == KVSEL_BF16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  } else {
    static_cast<uint16_t*>(p)[i] = f32_to_f16(v);
  }
}

// Order-preserving map of a finite float to uint32 (larger score -> larger
// key); -0.0 is folded onto +0.0 first.  Key 0 never arises from a finite
// value and marks "not a candidate".
__device__ __forceinline__ uint32_t score_key(float s) {
  // negative: every bit flipped; otherwise: the sign bit set
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 16-byte store marked non-temporal (global_store_dwordx4 ... nt): for outputs
// that the same launch never reads back, such as gathered or re-rotated K/V
// rows.  Streaming them past the caches keeps the write path at copy speed.
typedef unsigned int stream_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_stream(void* dst, const uint4& v) {
  __builtin_nontemporal_store(stream_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<stream_u32x4*>(dst));
}


// ---------------------------------------------------------------- launchers
// Each returns the status of the launch (hipGetLastError after enqueueing).

struct WindowParams {
  int L, Hq, Hkv, D, W, G;  // G = Hq / Hkv
  int64_t N;
  int causal;
  float scale;
  int head_agg, row_agg;
};

// VALU window passes.  lse == nullptr: the LSE pass leaves only its chunk
// partials, and the score pass, given them (partials != nullptr), merges
// each row's LSE itself (same bits as the combine); else it reads `lse`.
hipError_t launch_window_lse_valu(const WindowParams& p, int dt, const void* q, const void* k,
                                  float* partials, float* lse, hipStream_t st);
size_t window_valu_partials_bytes(const WindowParams& p);
hipError_t launch_window_scores_valu(const WindowParams& p, int dt, const void* q, const void* k,
                                     const float* lse, const float* partials, float* out, hipStream_t st);
bool window_mfma_supported(const WindowParams& p, int dt);
size_t window_mfma_partials_bytes(const WindowParams& p);
hipError_t launch_window_lse_mfma(const WindowParams& p, int dt, const void* q, const void* k,
                                  float* partials, float* lse, hipStream_t st);
hipError_t launch_window_scores_mfma(const WindowParams& p, int dt, const void* q, const void* k,
                                     const float* lse, float* out, hipStream_t st);

hipError_t launch_pool1d(const float* in, float* out, int64_t rows, int64_t n, int kind, int ksize,
                         hipStream_t st);

struct MemoryParams {
  int L, Hq, Hkv, D, page_size;
  int64_t N, pool_pages;
  int n_sink, n_recent;
  const int32_t* page_table;
  const int32_t* slot_map;
  int64_t dead_slot;
  float scale;
  int reduce;
};
// Memory-mode workspace: a fixed part (per-group LSE partials, LSE, per-layer
// rule rows) and a logit scratch of whole layers; the scratch the caller
// provides sets how many layers each pass covers (at least one).
size_t memory_fixed_bytes(const MemoryParams& p);
size_t memory_logit_bytes(const MemoryParams& p, bool minimum);
hipError_t launch_memory_scores(const MemoryParams& p, int dt, const float* M, const void* pool,
                                void* ws, float* logits, size_t logit_bytes, float* out, hipStream_t st);

// Packed tiles: a tile row is cut into chunks of kPackChunk columns; chunk c
// keeps the scores of its admitted columns, in ascending column order, at
// row positions [kPackChunk * c, kPackChunk * c + admitted), and admission
// masks of ceil(n / 64) words per row mark them (bit b of word w is column
// 64 w + b).
constexpr int kPackChunk = 256;

// Admission key of a threshold from kvsel_select's `admit` output: a column
// is admitted when score_key(score) > the key; NaN admits every column.
__device__ __forceinline__ uint32_t admit_key(float a) { return (a != a) ? 0u : score_key(a); }

struct BlockParams {
  int S, L, Hq, Hkv, D, W;
  int64_t NB, n_begin, n_count;
  float scale;
  const float* admit;     // [S][U] thresholds: packed output (D 128 only), or NULL: dense
  uint64_t* mask;         // [S][U][ceil(n_count / 64)] admission masks of the packed output
};
hipError_t launch_query_reduce(const BlockParams& p, int dt, const void* q, float* qbar,
                               hipStream_t st);
hipError_t launch_block_scores(const BlockParams& p, const float* qbar, const void* mu, float* out,
                               hipStream_t st);

struct SelectParams {
  int U;
  int64_t n, row_stride, base, n_total;
  int k_total, n_sink, n_recent;
  const int32_t* slot_map;
  int64_t dead_slot;
  float* cand_score;
  int32_t* cand_idx;
  int32_t* cand_count;
  int finalize;
  int32_t* kept_idx;
  uint8_t* keep_mask;
  int32_t* n_kept;
  int pool, pool_k;
  const uint64_t* tile_mask;  // tiled: admission masks of a packed tile, or NULL (dense)
  float* admit;               // tiled, not final: [U] admission threshold for the next tile, or NULL
};
// select_workspace_bytes(p): the keys and per-slice top-byte histograms of
// the two-launch paths (0 for the single-launch path and empty calls).
size_t select_workspace_bytes(const SelectParams& p);
// Tiled calls whose tile and running set fit in LDS run one launch of
// select_tile_kernel (no workspace).
bool select_tile_fits(const SelectParams& p);
hipError_t launch_select_tile(const SelectParams& p, const float* scores, hipStream_t st);
hipError_t launch_select(const SelectParams& p, const float* scores, void* ws, hipStream_t st);

struct RopeTable {
  double inv_freq[128];
};
struct GatherParams {
  int U, D, bt, k, dtype, rope, style, rotary_dim;
  int64_t src_unit_stride, src_rows, pos0, pool_pages;
  const int64_t* src_offsets;
  int64_t staged_cap;   // INCREMENTAL: >= 0 when misses come from packed staging (entries per unit)
  int hit_raw;          // INCREMENTAL: moved hits re-rotated from the raw source hit_src
  const void* hit_src;  //   (the raw K by block id, with src_offsets / src_unit_stride)
};
hipError_t launch_gather_fresh(const GatherParams& p, const RopeTable& rt, const void* src_k,
                               const void* src_v, const int32_t* idx, const int32_t* n_idx,
                               void* dst_k, void* dst_v, hipStream_t st);
size_t incremental_workspace_bytes(const GatherParams& p);
hipError_t launch_gather_incremental(const GatherParams& p, const RopeTable& rt, const void* src_k,
                                     const void* src_v, const int32_t* idx, const int32_t* prev_idx,
                                     const int32_t* prev_page, void* pool_k, void* pool_v,
                                     int32_t* page_table, int32_t* n_miss, void* ws,
                                     hipStream_t st);

struct IndexParams {
  int U, D, bt, dtype;
  int64_t src_unit_stride, src_rows, NB, b_begin, b_count;
  const int64_t* src_offsets;
};
hipError_t launch_build_index(const IndexParams& p, const void* src_k, uint16_t* mu, hipStream_t st);

// KVSEL_DEBUG=1 only: the number of NaN/Inf floats of x[rows][cols] (row
// stride `stride`); synchronises `st`.
hipError_t debug_count_nonfinite(const float* x, int64_t rows, int64_t cols, int64_t stride, hipStream_t st,
                                 uint64_t* count);
size_t free_list_workspace_bytes(int64_t n_slots);
hipError_t launch_free_list(int64_t N, const int32_t* slot_map, const uint8_t* keep, int64_t dead,
                            int64_t protected_len, int64_t n_slots, int32_t* free_slots, int32_t* n_free,
                            void* ws, hipStream_t st);
struct CompactParams {
  int R, L, Hkv, D, dtype, block_size, Y;
  int64_t N, pool_blocks;
};
size_t compact_workspace_bytes(const CompactParams& p);
hipError_t launch_compact(const CompactParams& p, const uint8_t* keep, const int32_t* block_table, void* k_pool,
                          void* v_pool, int32_t* slot_pos, int32_t* freed_blocks, int32_t* n_freed, void* ws,
                          hipStream_t st);

struct DecodeParams {
  int Ra, R, L, Hq, Hkv, D, G, block_size, Y;
  float scale2;   // softmax scale * log2(e)
  int64_t n_cap, pool_blocks;
  const int32_t* req;
  const int32_t* block_table;
  const int32_t* n_ctx;
  const int32_t* n_seen;
};
hipError_t launch_decode_score(const DecodeParams& p, int dt, const void* q, const float* lse, const void* k_pool,
                               float* state, hipStream_t st);

struct KeepScoreParams {
  int Rc, R, L, Hkv;
  int64_t n_cap;
  float lambda, top_p;
  const int32_t* req;
  const int32_t* n_len;
};
size_t keep_score_workspace_bytes(const KeepScoreParams& p, bool attn_given);
hipError_t launch_keep_score(const KeepScoreParams& p, const float* state, float* ks, float* attn_out,
                             uint8_t* hit, void* ws, hipStream_t st);

hipError_t launch_redirect(int64_t N, int32_t* slot_map, const uint8_t* keep, int64_t dead,
                           hipStream_t st);
// Redirect with the kept positions given as an ascending list (negative
// entries ignored): membership by binary search.
hipError_t launch_redirect_list(int64_t N, int32_t* slot_map, const int32_t* kept_idx, int32_t k, int64_t dead,
                                hipStream_t st);
hipError_t launch_sentinel(void* k_pool, void* v_pool, int L, int Hkv, int D, int dtype,
                           int64_t pool_slots, int64_t dead, hipStream_t st);
hipError_t launch_memory_update(int L, int Hq, int D, int W, int dt, const void* q, float* M,
                                float decay, hipStream_t st);

}  // namespace kvsel
