// C ABI of libkvsel: argument validation, workspace sizing and dispatch.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so argument errors are reported without a device.  Kernels
// are then enqueued on the caller's stream; nothing synchronises unless
// KVSEL_DEBUG=1.  No exception crosses the ABI.
#include <math.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace kvsel;

namespace {

thread_local std::string g_err;

kvsel_status fail(kvsel_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

kvsel_status hip_fail(hipError_t e, const char* what) {
  return fail(KVSEL_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool debug_mode() {
  static const bool on = [] {
    const char* v = getenv("KVSEL_DEBUG");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}

// KVSEL_DEBUG=1: NaN or Inf in a score array is reported as E_ARG.
kvsel_status debug_scores(const float* x, int64_t rows, int64_t cols, int64_t stride, hipStream_t st,
                          const char* what) {
  if (!debug_mode()) return KVSEL_OK;
  uint64_t bad = 0;
  const hipError_t e = debug_count_nonfinite(x, rows, cols, stride, st, &bad);
  if (e != hipSuccess) return hip_fail(e, "debug check");
  if (bad != 0)
    return fail(KVSEL_E_ARG, "%s hold %llu NaN or Inf values (inputs must be finite)", what,
                static_cast<unsigned long long>(bad));
  return KVSEL_OK;
}

// KVSEL_DEBUG=1: copies a small device index array to the host.
kvsel_status debug_fetch(const int32_t* d, size_t n, std::vector<int32_t>* h, hipStream_t st) {
  h->assign(n, 0);
  if (n == 0) return KVSEL_OK;
  hipError_t e = hipMemcpyAsync(h->data(), d, n * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  return (e == hipSuccess) ? KVSEL_OK : hip_fail(e, "debug check");
}

// KVSEL_DEBUG=1: the entries of v inside [0, limit) are pairwise distinct.
kvsel_status debug_distinct(const std::vector<int32_t>& v, int64_t limit, const char* what) {
  std::vector<int32_t> in;
  for (const int32_t x : v)
    if (x >= 0 && x < limit) in.push_back(x);
  std::sort(in.begin(), in.end());
  for (size_t i = 1; i < in.size(); ++i)
    if (in[i] == in[i - 1]) return fail(KVSEL_E_ARG, "%s: %d appears more than once", what, in[i]);
  return KVSEL_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == KVSEL_F32 || dt == KVSEL_BF16 || dt == KVSEL_F16; }
int dtype_size(int dt) { return dt == KVSEL_F32 ? 4 : 2; }
bool valid_agg(int a) { return a == KVSEL_AGG_SUM || a == KVSEL_AGG_MEAN || a == KVSEL_AGG_MAX; }

constexpr int64_t kMaxN = (int64_t(1) << 31) - 1;

// Per-device check that the device is gfx950 (cached).
kvsel_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::vector<int> state;   // 0 unknown, 1 ok, 2 unsupported
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<int>(state.size()) <= dev) state.resize(dev + 1, 0);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    if (state[dev] == 2) return fail(KVSEL_E_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (state[dev] == 2) return fail(KVSEL_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return KVSEL_OK;
}

kvsel_status finish(hipError_t e, hipStream_t st, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (debug_mode()) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, what);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, what);
  }
  g_err.clear();
  return KVSEL_OK;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// ------------------------------------------------------------------ score

struct ScorePlan {
  size_t lse_off = 0, part_off = 0, raw_off = 0, mem_off = 0, qbar_off = 0, total = 0;
  size_t logit_off = 0;   // memory mode: the logit scratch, last in the workspace
  size_t min_total = 0;   // the least workspace accepted (memory mode: one layer of logit scratch)
  bool mfma = false;
  bool own_lse = false;
  bool pooled = false;
  bool lse_only = false;
  const float* admit = nullptr;     // block mode, packed output
  uint64_t* tile_mask = nullptr;
};

kvsel_status validate_score(const kvsel_score_args* a, ScorePlan* plan) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < offsetof(kvsel_score_args, admit)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->mode < KVSEL_SCORE_WINDOW || a->mode > KVSEL_SCORE_BLOCK) return fail(KVSEL_E_ARG, "bad mode");
  if (a->struct_size >= sizeof(kvsel_score_args)) {
    plan->admit = a->admit;
    plan->tile_mask = a->tile_mask;
  }
  if ((plan->admit == nullptr) != (plan->tile_mask == nullptr))
    return fail(KVSEL_E_ARG, "give admit and tile_mask together (packed output) or neither");
  if (plan->admit != nullptr) {
    if (a->mode != KVSEL_SCORE_BLOCK) return fail(KVSEL_E_ARG, "admit and tile_mask are block-mode options");
    if (a->D != 128) return fail(KVSEL_E_UNSUPPORTED, "packed block scores need D = 128");
    if (!aligned16(plan->tile_mask)) return fail(KVSEL_E_ARG, "tile_mask must be 16-byte aligned");
  }
  if (a->L <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Hq % a->Hkv != 0)
    return fail(KVSEL_E_ARG, "need L, Hq, Hkv > 0 and Hkv dividing Hq");
  if (a->D != 64 && a->D != 128) return fail(KVSEL_E_UNSUPPORTED, "D must be 64 or 128");
  if (static_cast<int64_t>(a->L) * a->Hkv > 65535)
    return fail(KVSEL_E_UNSUPPORTED, "L * Hkv must be at most 65535 (one grid row per unit)");
  if (a->N <= 0 || a->N > kMaxN) return fail(KVSEL_E_ARG, "N must be in [1, 2^31)");
  const bool lse_only = a->mode == KVSEL_SCORE_WINDOW && a->scores == nullptr && a->lse_out != nullptr &&
                        a->lse_in == nullptr;
  if (a->scores == nullptr && !lse_only) return fail(KVSEL_E_ARG, "scores is NULL");
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->k_dtype)) return fail(KVSEL_E_ARG, "bad dtype");
  if (a->pool < KVSEL_POOL_NONE || a->pool > KVSEL_POOL_MAX) return fail(KVSEL_E_ARG, "bad pool");
  if (a->pool != KVSEL_POOL_NONE && (a->pool_k < 1 || a->pool_k % 2 == 0))
    return fail(KVSEL_E_ARG, "pool_k must be odd and >= 1");
  const int G = a->Hq / a->Hkv;
  const int U = a->L * a->Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round256(bytes);
    return o;
  };
  plan->pooled = a->pool != KVSEL_POOL_NONE && a->pool_k > 1 && !lse_only;
  plan->lse_only = lse_only;

  if (a->mode == KVSEL_SCORE_WINDOW) {
    if (a->q == nullptr || a->k == nullptr) return fail(KVSEL_E_ARG, "q or k is NULL");
    if (!aligned16(a->q) || !aligned16(a->k)) return fail(KVSEL_E_ARG, "q and k must be 16-byte aligned");
    if (a->q_dtype != a->k_dtype) return fail(KVSEL_E_UNSUPPORTED, "window mode needs q and k of one dtype");
    if (a->W < 1 || a->W > a->N) return fail(KVSEL_E_ARG, "W must be in [1, N]");
    if (!valid_agg(a->head_agg) || !valid_agg(a->row_agg)) return fail(KVSEL_E_ARG, "bad aggregation");
    WindowParams p{a->L, a->Hq, a->Hkv, a->D, a->W, G, a->N, a->causal ? 1 : 0, 1.f, a->head_agg, a->row_agg};
    plan->mfma = window_mfma_supported(p, a->k_dtype);
    if (!plan->mfma && static_cast<int64_t>(G) * a->W * a->D > 32768)
      return fail(KVSEL_E_UNSUPPORTED, "window of G*W*D > 32768 needs bf16/f16 with SUM/MEAN aggregation");
    plan->own_lse = a->lse_in == nullptr && a->lse_out == nullptr;
    if (plan->own_lse) plan->lse_off = take(static_cast<size_t>(a->L) * a->Hq * a->W * 4);
    if (a->lse_in == nullptr)
      plan->part_off = take(plan->mfma ? window_mfma_partials_bytes(p) : window_valu_partials_bytes(p));
    if (plan->pooled) plan->raw_off = take(static_cast<size_t>(U) * a->N * 4);
  } else if (a->mode == KVSEL_SCORE_MEMORY) {
    if (a->q == nullptr || a->k == nullptr || a->page_table == nullptr)
      return fail(KVSEL_E_ARG, "q (memory), k (pool) or page_table is NULL");
    if (!aligned16(a->k)) return fail(KVSEL_E_ARG, "pool must be 16-byte aligned");
    if (a->q_dtype != KVSEL_F32) return fail(KVSEL_E_UNSUPPORTED, "memory rows must be F32");
    if (a->k_dtype == KVSEL_F32) return fail(KVSEL_E_UNSUPPORTED, "memory mode needs a BF16/F16 pool");
    if (256 % a->Hq != 0) return fail(KVSEL_E_UNSUPPORTED, "memory mode needs Hq dividing 256");
    if (a->page_size < 1 || a->page_size > 64 || a->pool_pages < 1)
      return fail(KVSEL_E_ARG, "bad page_size or pool_pages");
    // the logits kernels stage two pages of every KV head in LDS (160 KiB per workgroup)
    if (2LL * a->page_size * a->Hkv * (2LL * a->D + 16) > 160 * 1024)
      return fail(KVSEL_E_UNSUPPORTED, "memory mode needs 2 * page_size * Hkv * (2 * D + 16) <= 160 KiB");
    if (a->n_sink < 0 || a->n_recent < 0) return fail(KVSEL_E_ARG, "negative forced-set size");
    if (a->reduce != KVSEL_REDUCE_GLOBAL && a->reduce != KVSEL_REDUCE_PER_UNIT)
      return fail(KVSEL_E_ARG, "bad reduce");
    MemoryParams mp{};
    mp.L = a->L; mp.Hq = a->Hq; mp.Hkv = a->Hkv; mp.D = a->D; mp.page_size = a->page_size;
    mp.N = a->N; mp.pool_pages = a->pool_pages;
    plan->mem_off = take(memory_fixed_bytes(mp));
    const int64_t rows = a->reduce == KVSEL_REDUCE_GLOBAL ? 1 : U;
    if (plan->pooled) plan->raw_off = take(static_cast<size_t>(rows) * a->N * 4);
    // the logit scratch comes last: a smaller workspace shortens only it
    plan->logit_off = take(memory_logit_bytes(mp, false));
    plan->min_total = plan->logit_off + memory_logit_bytes(mp, true);
  } else {
    if (a->k == nullptr) return fail(KVSEL_E_ARG, "index (k) is NULL");
    if (!aligned16(a->k)) return fail(KVSEL_E_ARG, "index must be 16-byte aligned");
    if (a->k_dtype != KVSEL_F16) return fail(KVSEL_E_UNSUPPORTED, "block mode needs an F16 Mean-K index");
    if (a->S < 1 || a->S > 8) return fail(KVSEL_E_ARG, "S must be in [1, 8]");
    if (a->n_begin < 0 || a->n_count < 0 || a->n_begin + a->n_count > a->N)
      return fail(KVSEL_E_ARG, "tile [n_begin, n_begin + n_count) outside [0, N)");
    if (a->qbar_valid) {
      if (a->qbar == nullptr) return fail(KVSEL_E_ARG, "qbar_valid with a NULL qbar");
    } else {
      if (a->q == nullptr) return fail(KVSEL_E_ARG, "q is NULL");
      if (!aligned16(a->q)) return fail(KVSEL_E_ARG, "q must be 16-byte aligned");
      if (a->W < 1) return fail(KVSEL_E_ARG, "W must be >= 1");
    }
    if (a->pool != KVSEL_POOL_NONE) return fail(KVSEL_E_UNSUPPORTED, "block mode has no pooling");
    if (a->qbar == nullptr) plan->qbar_off = take(static_cast<size_t>(a->S) * U * a->D * 4);
  }
  plan->total = off;
  if (plan->min_total == 0) plan->min_total = plan->total;
  return KVSEL_OK;
}

}  // namespace

extern "C" {

int32_t kvsel_version(void) { return KVSEL_ABI_VERSION; }

const char* kvsel_last_error(void) { return g_err.c_str(); }

kvsel_status kvsel_score_workspace(const kvsel_score_args* args, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    ScorePlan plan;
    kvsel_status s = validate_score(args, &plan);
    if (s != KVSEL_OK) return s;
    *bytes = plan.total;
    g_err.clear();
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_score(const kvsel_score_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    ScorePlan plan;
    kvsel_status s = validate_score(a, &plan);
    if (s != KVSEL_OK) return s;
    if (plan.total > 0 && (ws == nullptr || ws_bytes < plan.min_total))
      return fail(KVSEL_E_WORKSPACE, "workspace needs %zu bytes (at least %zu), got %zu", plan.total, plan.min_total,
                  ws == nullptr ? 0 : ws_bytes);
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* w = static_cast<uint8_t*>(ws);
    const float scale = (a->scale != 0.f) ? a->scale : static_cast<float>(1.0 / sqrt(static_cast<double>(a->D)));
    const int G = a->Hq / a->Hkv;
    const int U = a->L * a->Hkv;
    hipError_t e = hipSuccess;
    float* dst = plan.pooled ? reinterpret_cast<float*>(w + plan.raw_off) : a->scores;
    int64_t pool_rows = U;

    if (a->mode == KVSEL_SCORE_WINDOW) {
      WindowParams p{a->L, a->Hq, a->Hkv, a->D, a->W, G, a->N, a->causal ? 1 : 0, scale,
                     a->head_agg, a->row_agg};
      const float* lse = a->lse_in;
      // the VALU score pass merges the LSE partials itself when the caller
      // asks for no LSE output (one launch fewer)
      const bool fuse_lse = !plan.mfma && lse == nullptr && plan.own_lse && !plan.lse_only;
      const float* part = reinterpret_cast<const float*>(w + plan.part_off);
      if (lse == nullptr) {
        float* lo = plan.own_lse ? reinterpret_cast<float*>(w + plan.lse_off) : a->lse_out;
        if (plan.mfma)
          e = launch_window_lse_mfma(p, a->k_dtype, a->q, a->k, reinterpret_cast<float*>(w + plan.part_off), lo, st);
        else
          e = launch_window_lse_valu(p, a->k_dtype, a->q, a->k, reinterpret_cast<float*>(w + plan.part_off),
                                     fuse_lse ? nullptr : lo, st);
        if (e != hipSuccess) return hip_fail(e, "window lse");
        lse = lo;
      }
      if (plan.lse_only) return finish(hipSuccess, st, "window lse");
      if (plan.mfma) e = launch_window_scores_mfma(p, a->k_dtype, a->q, a->k, lse, dst, st);
      else e = launch_window_scores_valu(p, a->k_dtype, a->q, a->k, lse, fuse_lse ? part : nullptr, dst, st);
      if (e != hipSuccess) return hip_fail(e, "window scores");
    } else if (a->mode == KVSEL_SCORE_MEMORY) {
      MemoryParams p{};
      p.L = a->L; p.Hq = a->Hq; p.Hkv = a->Hkv; p.D = a->D; p.page_size = a->page_size;
      p.N = a->N; p.pool_pages = a->pool_pages; p.n_sink = a->n_sink; p.n_recent = a->n_recent;
      p.page_table = a->page_table; p.slot_map = a->slot_map; p.dead_slot = a->dead_slot;
      p.scale = scale; p.reduce = a->reduce;
      e = launch_memory_scores(p, a->k_dtype, static_cast<const float*>(a->q), a->k, w + plan.mem_off,
                               reinterpret_cast<float*>(w + plan.logit_off), ws_bytes - plan.logit_off, dst, st);
      if (e != hipSuccess) return hip_fail(e, "memory scores");
      pool_rows = (a->reduce == KVSEL_REDUCE_GLOBAL) ? 1 : U;
    } else {
      BlockParams p{a->S, a->L, a->Hq, a->Hkv, a->D, a->W, a->N, a->n_begin, a->n_count, scale,
                    plan.admit, plan.tile_mask};
      float* qbar = a->qbar ? a->qbar : reinterpret_cast<float*>(w + plan.qbar_off);
      if (!a->qbar_valid) {
        e = launch_query_reduce(p, a->q_dtype, a->q, qbar, st);
        if (e != hipSuccess) return hip_fail(e, "query reduce");
      }
      e = launch_block_scores(p, qbar, a->k, a->scores, st);
      if ((s = finish(e, st, "block scores")) != KVSEL_OK) return s;
      if (plan.admit != nullptr) return KVSEL_OK;   // packed rows hold unwritten positions
      return debug_scores(a->scores, static_cast<int64_t>(a->S) * U, a->n_count, a->n_count, st,
                          "block scores (q or the index not finite?)");
    }
    if (plan.pooled) e = launch_pool1d(dst, a->scores, pool_rows, a->N, a->pool, a->pool_k, st);
    if ((s = finish(e, st, "score pooling")) != KVSEL_OK) return s;
    return debug_scores(a->scores, pool_rows, a->N, a->N, st, "scores (q, k or lse_in not finite?)");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ select

static kvsel_status validate_select(const kvsel_select_args* a) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < offsetof(kvsel_select_args, tile_mask)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->U < 0 || a->n < 0 || a->base < 0 || a->k_total < 0 || a->n_sink < 0 || a->n_recent < 0)
    return fail(KVSEL_E_ARG, "negative size");
  if (a->n_total > kMaxN || a->base + a->n > a->n_total)
    return fail(KVSEL_E_ARG, "need base + n <= n_total < 2^31");
  if (a->U > 65535) return fail(KVSEL_E_UNSUPPORTED, "U must be at most 65535 (one grid row per unit)");
  if (a->U > 0 && a->n > 0 && (a->scores == nullptr || a->row_stride < a->n))
    return fail(KVSEL_E_ARG, "scores NULL or row_stride < n");
  if (a->k_total < a->n_total && static_cast<int64_t>(a->n_sink) + a->n_recent > a->k_total)
    return fail(KVSEL_E_BUDGET, "n_sink + n_recent (%d) exceeds k_total (%d) < n_total", a->n_sink + a->n_recent,
                a->k_total);
  const int ncand = (a->cand_score != nullptr) + (a->cand_idx != nullptr) + (a->cand_count != nullptr);
  if (ncand != 0 && ncand != 3) return fail(KVSEL_E_ARG, "give all of cand_score, cand_idx, cand_count or none");
  const bool tiled = ncand == 3;
  if (!tiled && (a->base != 0 || a->n != a->n_total))
    return fail(KVSEL_E_ARG, "a partial range needs the running-candidate buffers");
  if (!tiled && !a->finalize) return fail(KVSEL_E_ARG, "an untiled call must finalize");
  if (a->keep_mask != nullptr && (tiled || a->base != 0 || a->n != a->n_total))
    return fail(KVSEL_E_ARG, "keep_mask needs an untiled call");
  if (a->U > 0 && a->finalize && a->kept_idx == nullptr) return fail(KVSEL_E_ARG, "kept_idx is NULL");
  if (a->pool < KVSEL_POOL_NONE || a->pool > KVSEL_POOL_MAX) return fail(KVSEL_E_ARG, "bad pool");
  if (a->pool != KVSEL_POOL_NONE && (a->pool_k < 1 || a->pool_k % 2 == 0 || a->pool_k > 255))
    return fail(KVSEL_E_ARG, "pool_k must be odd, in [1, 255]");
  if (a->pool != KVSEL_POOL_NONE && tiled) return fail(KVSEL_E_ARG, "pooling needs an untiled call");
  if (tiled && static_cast<int64_t>(a->k_total) * 8 > 64 * 1024)
    return fail(KVSEL_E_UNSUPPORTED, "tiled selection supports k_total <= 8192");
  if (a->struct_size >= sizeof(kvsel_select_args) && (a->tile_mask != nullptr || a->admit != nullptr)) {
    if (!tiled) return fail(KVSEL_E_ARG, "tile_mask and admit need a tiled call");
    if (!aligned16(a->tile_mask) || !aligned16(a->admit))
      return fail(KVSEL_E_ARG, "tile_mask and admit must be 16-byte aligned");
    // both live in the one-launch tile kernel only
    SelectParams p{};
    p.U = a->U; p.n = a->n; p.k_total = a->k_total; p.cand_count = a->cand_count;
    if (!select_tile_fits(p))
      return fail(KVSEL_E_UNSUPPORTED, "tile_mask and admit need a tile call that fits one workgroup's LDS");
  }
  return KVSEL_OK;
}

static SelectParams select_params(const kvsel_select_args* a) {
  SelectParams p{};
  p.U = a->U; p.n = a->n; p.row_stride = a->row_stride; p.base = a->base; p.n_total = a->n_total;
  p.k_total = a->k_total; p.n_sink = a->n_sink; p.n_recent = a->n_recent;
  p.slot_map = a->slot_map; p.dead_slot = a->dead_slot;
  p.cand_score = a->cand_score; p.cand_idx = a->cand_idx; p.cand_count = a->cand_count;
  p.finalize = a->finalize ? 1 : 0;
  if (a->cand_count == nullptr) p.finalize = 1;
  p.kept_idx = a->kept_idx; p.keep_mask = a->keep_mask; p.n_kept = a->n_kept;
  p.pool = (a->pool_k > 1) ? a->pool : KVSEL_POOL_NONE;
  p.pool_k = a->pool_k;
  if (a->struct_size >= sizeof(kvsel_select_args)) {
    p.tile_mask = a->tile_mask;
    p.admit = a->admit;
  }
  return p;
}

kvsel_status kvsel_select_workspace(const kvsel_select_args* a, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    kvsel_status s = validate_select(a);
    if (s != KVSEL_OK) return s;
    *bytes = select_workspace_bytes(select_params(a));
    g_err.clear();
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_select(const kvsel_select_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    kvsel_status s = validate_select(a);
    if (s != KVSEL_OK) return s;
    const SelectParams p = select_params(a);
    const size_t need = select_workspace_bytes(p);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(KVSEL_E_WORKSPACE, "select needs %zu bytes of workspace, got %zu", need, ws == nullptr ? 0 : ws_bytes);
    if (need > 0 && !aligned16(ws)) return fail(KVSEL_E_ARG, "workspace must be 16-byte aligned");
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.U > 0 && p.n > 0 && p.tile_mask == nullptr &&
        (s = debug_scores(a->scores, p.U, p.n, p.row_stride, st, "scores")) != KVSEL_OK)
      return s;
    return finish(launch_select(p, a->scores, ws, st), st, "select");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ select, no allocation
//
// For callers that cannot allocate device memory: the select workspace lives
// in a fixed array of the library, one per device, instead of a caller
// buffer.  Host code never uses the array's name as an address (that is a
// host-side stand-in); it resolves the device address once per device with
// hipGetSymbolAddress and passes that pointer to the kernels.

namespace {

static __device__ __align__(256) unsigned char scratch[KVSEL_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, resolved on the first
// call per device (with that device current) and kept for the process.
kvsel_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  static std::mutex mu;
  static std::vector<void*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<int>(ptrs.size()) <= dev) ptrs.resize(dev + 1, nullptr);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(KVSEL_E_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return KVSEL_OK;
}

}  // namespace

kvsel_status kvsel_select_noalloc(const kvsel_select_args* a, void* stream) {
  try {
    kvsel_status s = validate_select(a);
    if (s != KVSEL_OK) return s;
    const SelectParams p = select_params(a);
    const size_t need = select_workspace_bytes(p);
    if (need > static_cast<size_t>(KVSEL_NOALLOC_SCRATCH_BYTES))
      return fail(KVSEL_E_WORKSPACE, "select needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                  static_cast<size_t>(KVSEL_NOALLOC_SCRATCH_BYTES));
    if ((s = check_device()) != KVSEL_OK) return s;
    void* ws = nullptr;
    if (need > 0 && (s = noalloc_scratch(&ws)) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.U > 0 && p.n > 0 && p.tile_mask == nullptr &&
        (s = debug_scores(a->scores, p.U, p.n, p.row_stride, st, "scores")) != KVSEL_OK)
      return s;
    // every word of the scratch a launch reads is written earlier in the
    // same call (keys and per-slice histograms), so nothing is cleared
    return finish(launch_select(p, a->scores, ws, st), st, "select (no allocation)");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ gather

// The packed-miss fields were appended to kvsel_gather_args; a struct that
// ends before them is the raw-source form.
struct GatherStaging {
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t cap = 0;
  int hit_raw = 0;
};

static GatherStaging gather_staging(const kvsel_gather_args* a) {
  GatherStaging g;
  if (a->struct_size >= sizeof(kvsel_gather_args)) {
    g.k = a->staged_k;
    g.v = a->staged_v;
    g.cap = a->staged_cap;
    g.hit_raw = a->hit_raw;
  }
  return g;
}

static kvsel_status validate_gather(const kvsel_gather_args* a, GatherParams* gp, RopeTable* rt) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < offsetof(kvsel_gather_args, staged_k)) return fail(KVSEL_E_ARG, "struct_size too small");
  const GatherStaging stg = gather_staging(a);
  const bool staged = a->mode == KVSEL_GATHER_INCREMENTAL && stg.k != nullptr;
  if (a->mode != KVSEL_GATHER_FRESH && a->mode != KVSEL_GATHER_INCREMENTAL) return fail(KVSEL_E_ARG, "bad mode");
  if (!valid_dtype(a->dtype)) return fail(KVSEL_E_ARG, "bad dtype");
  if (a->U < 0 || a->k < 0 || a->bt < 1) return fail(KVSEL_E_ARG, "need U, k >= 0 and bt >= 1");
  const int esz = dtype_size(a->dtype);
  const int elems16 = 16 / esz;
  const int lpr = (a->D > 0) ? a->D * esz / 16 : 0;
  if (a->D <= 0 || (a->D * esz) % 16 != 0 || lpr > 64 || (lpr & (lpr - 1)) != 0)
    return fail(KVSEL_E_UNSUPPORTED, "D*elem_size must be 16 * a power of two <= 1024 bytes");
  if (a->rope < KVSEL_ROPE_NONE || a->rope > KVSEL_ROPE_DELTA) return fail(KVSEL_E_ARG, "bad rope");
  const int rd = a->rotary_dim == 0 ? a->D : a->rotary_dim;
  if (a->rope != KVSEL_ROPE_NONE) {
    if (a->style != KVSEL_ROPE_HALF && a->style != KVSEL_ROPE_INTERLEAVED) return fail(KVSEL_E_ARG, "bad style");
    if (rd < 2 || rd > a->D || rd % 2 != 0) return fail(KVSEL_E_ARG, "bad rotary_dim");
    const int need = (a->style == KVSEL_ROPE_HALF) ? 2 * elems16 : elems16;
    if (rd % need != 0) return fail(KVSEL_E_UNSUPPORTED, "rotary_dim must be a multiple of %d", need);
    if (rd / 2 > 128) return fail(KVSEL_E_UNSUPPORTED, "rotary_dim must be <= 256");
    if (!(a->theta > 0.0)) return fail(KVSEL_E_ARG, "theta must be > 0");
  }
  if (a->idx == nullptr) return fail(KVSEL_E_ARG, "idx is NULL");
  if (stg.hit_raw != 0 && stg.hit_raw != 1) return fail(KVSEL_E_ARG, "hit_raw must be 0 or 1");
  const bool hit_raw = a->mode == KVSEL_GATHER_INCREMENTAL && stg.hit_raw == 1;
  if (hit_raw && (a->src_k == nullptr || !aligned16(a->src_k)))
    return fail(KVSEL_E_ARG, "hit_raw needs src_k (16-byte aligned) to re-rotate moved hits from");
  if (staged) {
    if (stg.v == nullptr) return fail(KVSEL_E_ARG, "staged_v is NULL");
    if (!aligned16(stg.k) || !aligned16(stg.v)) return fail(KVSEL_E_ARG, "staging buffers must be 16-byte aligned");
    if (stg.cap < 0) return fail(KVSEL_E_ARG, "staged_cap < 0");
  } else {
    if (a->src_k == nullptr || a->src_v == nullptr) return fail(KVSEL_E_ARG, "src_k or src_v is NULL");
    if (!aligned16(a->src_k) || !aligned16(a->src_v)) return fail(KVSEL_E_ARG, "sources must be 16-byte aligned");
  }
  if (a->src_rows < 0) return fail(KVSEL_E_ARG, "src_rows < 0");
  if (a->mode == KVSEL_GATHER_FRESH) {
    if (a->dst_k == nullptr || a->dst_v == nullptr) return fail(KVSEL_E_ARG, "dst_k or dst_v is NULL");
    if (!aligned16(a->dst_k) || !aligned16(a->dst_v)) return fail(KVSEL_E_ARG, "destinations must be 16-byte aligned");
  } else {
    if (a->prev_idx == nullptr || a->prev_page == nullptr || a->pool_k == nullptr || a->pool_v == nullptr ||
        a->page_table == nullptr || a->n_miss == nullptr)
      return fail(KVSEL_E_ARG, "incremental mode needs prev_idx, prev_page, pools, page_table, n_miss");
    if (!aligned16(a->pool_k) || !aligned16(a->pool_v)) return fail(KVSEL_E_ARG, "pools must be 16-byte aligned");
    if (a->pool_pages < a->k) return fail(KVSEL_E_ARG, "pool_pages < k");
    if (a->rope == KVSEL_ROPE_DELTA) return fail(KVSEL_E_ARG, "incremental mode rotates raw K (rope RAW or NONE)");
    if (a->k > 8192 || a->pool_pages > (int64_t(1) << 18))
      return fail(KVSEL_E_UNSUPPORTED, "incremental mode supports k <= 8192 and pool_pages <= 2^18");
    if (a->rope == KVSEL_ROPE_RAW && (rd != a->D || static_cast<int64_t>(a->bt) * (a->D / 2) > 2048))
      return fail(KVSEL_E_UNSUPPORTED, "incremental re-RoPE needs rotary_dim == D and bt * D/2 <= 2048");
  }
  gp->U = a->U; gp->D = a->D; gp->bt = a->bt; gp->k = a->k; gp->dtype = a->dtype; gp->rope = a->rope;
  gp->style = a->style; gp->rotary_dim = rd; gp->src_unit_stride = a->src_unit_stride;
  gp->src_rows = a->src_rows; gp->pos0 = a->pos0; gp->pool_pages = a->pool_pages; gp->src_offsets = a->src_offsets;
  gp->staged_cap = staged ? stg.cap : -1;
  gp->hit_raw = hit_raw ? 1 : 0;
  gp->hit_src = hit_raw ? a->src_k : nullptr;
  for (int m = 0; m < 128; ++m) rt->inv_freq[m] = (m < rd / 2) ? pow(a->theta, -2.0 * m / rd) : 0.0;
  return KVSEL_OK;
}

kvsel_status kvsel_gather_workspace(const kvsel_gather_args* a, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    GatherParams gp{};
    RopeTable rt;
    kvsel_status s = validate_gather(a, &gp, &rt);
    if (s != KVSEL_OK) return s;
    *bytes = (a->mode == KVSEL_GATHER_INCREMENTAL) ? incremental_workspace_bytes(gp) : 0;
    g_err.clear();
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// KVSEL_DEBUG=1: the in-place view update relies on ascending, valid block
// lists and on distinct pages per unit; a violation would race silently.
static kvsel_status debug_incremental(const kvsel_gather_args* a, hipStream_t st) {
  const size_t n = static_cast<size_t>(a->U) * a->k;
  std::vector<int32_t> idx, prev, page;
  kvsel_status s;
  if ((s = debug_fetch(a->idx, n, &idx, st)) != KVSEL_OK || (s = debug_fetch(a->prev_idx, n, &prev, st)) != KVSEL_OK ||
      (s = debug_fetch(a->prev_page, n, &page, st)) != KVSEL_OK)
    return s;
  // with packed staging the block ids address no source, so any id is valid
  const int64_t blocks = (gather_staging(a).k != nullptr) ? (int64_t(1) << 31) : a->src_rows / a->bt;
  for (int u = 0; u < a->U; ++u) {
    for (int i = 0; i < a->k; ++i) {
      const size_t o = static_cast<size_t>(u) * a->k + i;
      if (idx[o] < 0 || idx[o] >= blocks || (i > 0 && idx[o] <= idx[o - 1]))
        return fail(KVSEL_E_ARG, "idx of unit %d is not ascending within [0, %lld) at %d", u,
                    static_cast<long long>(blocks), i);
      if (prev[o] < 0 || (i > 0 && prev[o] <= prev[o - 1]))
        return fail(KVSEL_E_ARG, "prev_idx of unit %d is not ascending and valid at %d", u, i);
      if (page[o] < 0 || page[o] >= a->pool_pages)
        return fail(KVSEL_E_ARG, "prev_page of unit %d is outside [0, pool_pages) at %d", u, i);
    }
    const std::vector<int32_t> row(page.begin() + static_cast<size_t>(u) * a->k,
                                   page.begin() + static_cast<size_t>(u + 1) * a->k);
    if ((s = debug_distinct(row, a->pool_pages, "prev_page")) != KVSEL_OK) return s;
  }
  return KVSEL_OK;
}

kvsel_status kvsel_gather_rerope(const kvsel_gather_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    GatherParams gp{};
    RopeTable rt;
    kvsel_status s = validate_gather(a, &gp, &rt);
    if (s != KVSEL_OK) return s;
    const size_t need = (a->mode == KVSEL_GATHER_INCREMENTAL) ? incremental_workspace_bytes(gp) : 0;
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(KVSEL_E_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_mode() && a->mode == KVSEL_GATHER_INCREMENTAL && (s = debug_incremental(a, st)) != KVSEL_OK) return s;
    hipError_t e;
    if (a->mode == KVSEL_GATHER_FRESH)
      e = launch_gather_fresh(gp, rt, a->src_k, a->src_v, a->idx, a->n_idx, a->dst_k, a->dst_v, st);
    else
      e = launch_gather_incremental(gp, rt, gp.staged_cap >= 0 ? gather_staging(a).k : a->src_k,
                                    gp.staged_cap >= 0 ? gather_staging(a).v : a->src_v, a->idx, a->prev_idx,
                                    a->prev_page, a->pool_k, a->pool_v, a->page_table, a->n_miss, ws, st);
    return finish(e, st, "gather");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ redirect

kvsel_status kvsel_redirect(const kvsel_redirect_args* a, void* stream) {
  try {
    if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
    if (a->struct_size < offsetof(kvsel_redirect_args, kept_idx)) return fail(KVSEL_E_ARG, "struct_size too small");
    // the kept-index form was appended; a struct ending before it has only the mask form
    const bool list_form = a->struct_size >= sizeof(kvsel_redirect_args) && a->keep_mask == nullptr;
    const int32_t* kept_idx = list_form ? a->kept_idx : nullptr;
    const int32_t n_list = list_form ? a->k : 0;
    if (a->N < 0 || a->N > kMaxN) return fail(KVSEL_E_ARG, "N must be in [0, 2^31)");
    if (a->N > 0 && a->slot_map == nullptr) return fail(KVSEL_E_ARG, "slot_map is NULL");
    if (a->N > 0 && a->keep_mask == nullptr && !(list_form && (kept_idx != nullptr || n_list == 0)))
      return fail(KVSEL_E_ARG, "give keep_mask, or kept_idx with k");
    if (list_form && n_list < 0) return fail(KVSEL_E_ARG, "k < 0");
    if (a->dead_slot < 0 || a->dead_slot > kMaxN) return fail(KVSEL_E_ARG, "dead_slot outside int32");
    const bool sentinel = a->k_pool != nullptr;
    if (sentinel) {
      if (a->v_pool == nullptr) return fail(KVSEL_E_ARG, "v_pool is NULL");
      if (a->dtype != KVSEL_BF16 && a->dtype != KVSEL_F16)
        return fail(KVSEL_E_UNSUPPORTED, "the sentinel needs a BF16/F16 pool (-1e4 is not an fp8 value)");
      if (a->L <= 0 || a->Hkv <= 0 || a->D <= 0 || a->pool_slots <= a->dead_slot)
        return fail(KVSEL_E_ARG, "bad pool shape or dead_slot outside the pool");
    }
    kvsel_status s = check_device();
    if (s != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_mode() && list_form && n_list > 0) {
      std::vector<int32_t> h;
      if ((s = debug_fetch(kept_idx, static_cast<size_t>(n_list), &h, st)) != KVSEL_OK) return s;
      for (int32_t i = 1; i < n_list && h[i] >= 0; ++i)
        if (h[i] <= h[i - 1]) return fail(KVSEL_E_ARG, "kept_idx is not ascending at %d", i);
      for (int32_t i = 1; i < n_list; ++i)
        if (h[i - 1] < 0 && h[i] >= 0) return fail(KVSEL_E_ARG, "kept_idx has a valid entry after a negative one at %d", i);
    }
    hipError_t e = hipSuccess;
    if (sentinel) {
      e = launch_sentinel(a->k_pool, a->v_pool, a->L, a->Hkv, a->D, a->dtype, a->pool_slots, a->dead_slot, st);
      if (e != hipSuccess) return hip_fail(e, "sentinel");
    }
    e = list_form ? launch_redirect_list(a->N, a->slot_map, kept_idx, n_list, a->dead_slot, st)
                  : launch_redirect(a->N, a->slot_map, a->keep_mask, a->dead_slot, st);
    return finish(e, st, "redirect");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ memory

static kvsel_status check_compact(const kvsel_compact_args* a, CompactParams* p) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < sizeof(kvsel_compact_args)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->R < 0 || a->Y < 0) return fail(KVSEL_E_ARG, "R and Y must be >= 0");
  if (a->R > 65535) return fail(KVSEL_E_UNSUPPORTED, "R must be at most 65535 (one grid row per request)");
  if (a->L < 1 || a->Hkv < 1 || a->D < 1 || a->block_size < 1 || a->pool_blocks < 1)
    return fail(KVSEL_E_ARG, "L, Hkv, D, block_size and pool_blocks must be >= 1");
  if (!valid_dtype(a->dtype)) return fail(KVSEL_E_ARG, "bad dtype");
  const int64_t slots = static_cast<int64_t>(a->Y) * a->block_size;
  if (slots > kMaxN) return fail(KVSEL_E_ARG, "Y * block_size must be below 2^31");
  if (a->N < 0 || a->N > slots) return fail(KVSEL_E_ARG, "N must be in [0, Y * block_size]");
  const int esz = (a->dtype == KVSEL_F32) ? 4 : 2;
  if ((static_cast<int64_t>(a->Hkv) * a->D * esz) % 16 != 0)
    return fail(KVSEL_E_ARG, "Hkv * D * element size must be a multiple of 16 bytes");
  if (a->R > 0 && a->Y > 0) {
    if (a->keep_mask == nullptr || a->block_table == nullptr || a->k_pool == nullptr || a->v_pool == nullptr ||
        a->slot_pos == nullptr || a->freed_blocks == nullptr || a->n_freed == nullptr)
      return fail(KVSEL_E_ARG, "a pointer is NULL");
    if (!aligned16(a->k_pool) || !aligned16(a->v_pool)) return fail(KVSEL_E_ARG, "pools must be 16-byte aligned");
    const uintptr_t mis = reinterpret_cast<uintptr_t>(a->block_table) | reinterpret_cast<uintptr_t>(a->slot_pos) |
                          reinterpret_cast<uintptr_t>(a->freed_blocks) | reinterpret_cast<uintptr_t>(a->n_freed);
    if ((mis & 3u) != 0) return fail(KVSEL_E_ARG, "int32 arrays must be 4-byte aligned");
  }
  p->R = a->R; p->L = a->L; p->Hkv = a->Hkv; p->D = a->D; p->dtype = a->dtype;
  p->block_size = a->block_size; p->Y = a->Y; p->N = a->N; p->pool_blocks = a->pool_blocks;
  return KVSEL_OK;
}

kvsel_status kvsel_compact_workspace(const kvsel_compact_args* a, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    CompactParams p;
    kvsel_status s = check_compact(a, &p);
    if (s != KVSEL_OK) return s;
    *bytes = compact_workspace_bytes(p);
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_compact(const kvsel_compact_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    CompactParams p;
    kvsel_status s = check_compact(a, &p);
    if (s != KVSEL_OK) return s;
    if (p.R == 0 || p.Y == 0) return KVSEL_OK;
    const size_t need = compact_workspace_bytes(p);
    if (ws == nullptr || ws_bytes < need) return fail(KVSEL_E_WORKSPACE, "workspace too small (see kvsel_compact_workspace)");
    if (!aligned16(ws)) return fail(KVSEL_E_ARG, "workspace must be 16-byte aligned");
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_mode()) {
      std::vector<int32_t> bt;
      if ((s = debug_fetch(a->block_table, static_cast<size_t>(a->R) * a->Y, &bt, st)) != KVSEL_OK ||
          (s = debug_distinct(bt, a->pool_blocks, "block_table")) != KVSEL_OK)
        return s;
    }
    return finish(launch_compact(p, a->keep_mask, a->block_table, a->k_pool, a->v_pool, a->slot_pos,
                                 a->freed_blocks, a->n_freed, ws, st),
                  st, "compaction");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

static kvsel_status check_free_list(const kvsel_freelist_args* a) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < sizeof(kvsel_freelist_args)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->N < 0 || a->N > kMaxN) return fail(KVSEL_E_ARG, "N must be in [0, 2^31)");
  if (a->n_slots < 1 || a->n_slots > kMaxN) return fail(KVSEL_E_ARG, "n_slots must be in [1, 2^31)");
  if (a->protected_len < 0) return fail(KVSEL_E_ARG, "protected_len must be >= 0");
  if (a->n_free == nullptr) return fail(KVSEL_E_ARG, "n_free is NULL");
  if (a->N > 0 && (a->slot_map == nullptr || a->keep_mask == nullptr || a->free_slots == nullptr))
    return fail(KVSEL_E_ARG, "slot_map, keep_mask or free_slots is NULL");
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a->slot_map) | reinterpret_cast<uintptr_t>(a->free_slots) |
                        reinterpret_cast<uintptr_t>(a->n_free);
  if ((mis & 3u) != 0) return fail(KVSEL_E_ARG, "slot_map, free_slots and n_free must be 4-byte aligned");
  return KVSEL_OK;
}

kvsel_status kvsel_free_list_workspace(const kvsel_freelist_args* a, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    kvsel_status s = check_free_list(a);
    if (s != KVSEL_OK) return s;
    *bytes = free_list_workspace_bytes(a->n_slots);
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_free_list(const kvsel_freelist_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    kvsel_status s = check_free_list(a);
    if (s != KVSEL_OK) return s;
    const size_t need = free_list_workspace_bytes(a->n_slots);
    if (ws == nullptr || ws_bytes < need) return fail(KVSEL_E_WORKSPACE, "workspace too small (see kvsel_free_list_workspace)");
    if (!aligned16(ws)) return fail(KVSEL_E_ARG, "workspace must be 16-byte aligned");
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(launch_free_list(a->N, a->slot_map, a->keep_mask, a->dead_slot, a->protected_len, a->n_slots,
                                   a->free_slots, a->n_free, ws, st),
                  st, "free list");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_build_index(const kvsel_index_args* a, void* stream) {
  try {
    if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
    if (a->struct_size < sizeof(kvsel_index_args)) return fail(KVSEL_E_ARG, "struct_size too small");
    if (a->U < 0) return fail(KVSEL_E_ARG, "U must be >= 0");
    if (!valid_dtype(a->dtype)) return fail(KVSEL_E_ARG, "bad dtype");
    if (a->D != 64 && a->D != 128) return fail(KVSEL_E_UNSUPPORTED, "D must be 64 or 128");
    if (a->bt < 1 || a->bt > 256) return fail(KVSEL_E_ARG, "bt must be in [1, 256]");
    if (a->NB < 0 || a->b_begin < 0 || a->b_count < 0 || a->b_begin + a->b_count > a->NB)
      return fail(KVSEL_E_ARG, "need 0 <= b_begin, 0 <= b_count, b_begin + b_count <= NB");
    if ((a->b_begin + a->b_count) * a->bt > a->src_rows)
      return fail(KVSEL_E_ARG, "the block range reaches past src_rows");
    if (a->U == 0 || a->b_count == 0) return KVSEL_OK;
    if (a->src_k == nullptr || a->mu == nullptr) return fail(KVSEL_E_ARG, "src_k or mu is NULL");
    const int esz = (a->dtype == KVSEL_F32) ? 4 : 2;
    if (!aligned16(a->src_k) || !aligned16(a->mu)) return fail(KVSEL_E_ARG, "src_k and mu must be 16-byte aligned");
    if (a->src_offsets == nullptr && (a->src_unit_stride < 0 || (a->src_unit_stride * esz) % 16 != 0))
      return fail(KVSEL_E_ARG, "src_unit_stride must be >= 0 and keep units 16-byte aligned");
    kvsel_status s = check_device();
    if (s != KVSEL_OK) return s;
    IndexParams p;
    p.U = a->U; p.D = a->D; p.bt = a->bt; p.dtype = a->dtype;
    p.src_unit_stride = a->src_unit_stride; p.src_rows = a->src_rows; p.NB = a->NB;
    p.b_begin = a->b_begin; p.b_count = a->b_count; p.src_offsets = a->src_offsets;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(launch_build_index(p, a->src_k, a->mu, st), st, "index build");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_memory_update(const kvsel_memupd_args* a, void* stream) {
  try {
    if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
    if (a->struct_size < sizeof(kvsel_memupd_args)) return fail(KVSEL_E_ARG, "struct_size too small");
    if (a->L <= 0 || a->Hq <= 0 || a->D <= 0 || a->D > 256 || a->W <= 0)
      return fail(KVSEL_E_ARG, "need L, Hq, W > 0 and 0 < D <= 256");
    if (a->q_turn == nullptr || a->M == nullptr) return fail(KVSEL_E_ARG, "q_turn or M is NULL");
    if (!valid_dtype(a->q_dtype)) return fail(KVSEL_E_ARG, "bad dtype");
    kvsel_status s = check_device();
    if (s != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(launch_memory_update(a->L, a->Hq, a->D, a->W, a->q_dtype, a->q_turn, a->M, a->decay, st), st,
                  "memory update");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

}  // extern "C"

// ------------------------------------------------------------------ decode scorer

static kvsel_status check_decode(const kvsel_decode_args* a, DecodeParams* p) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < sizeof(kvsel_decode_args)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->Ra < 0 || a->R < 0 || a->Ra > 65535) return fail(KVSEL_E_ARG, "Ra must be in [0, 65535] and R >= 0");
  if (a->L < 1 || a->L > 65535 || a->Hq < 1 || a->Hkv < 1 || a->block_size < 1 || a->Y < 0 || a->pool_blocks < 1)
    return fail(KVSEL_E_ARG, "L in [1, 65535], Hq, Hkv, block_size, pool_blocks >= 1 and Y >= 0 required");
  if (a->dtype != KVSEL_BF16 && a->dtype != KVSEL_F16) return fail(KVSEL_E_UNSUPPORTED, "dtype must be BF16 or F16");
  if (a->D != 64 && a->D != 128) return fail(KVSEL_E_UNSUPPORTED, "D must be 64 or 128");
  if (a->Hq % a->Hkv != 0) return fail(KVSEL_E_ARG, "Hq must be a multiple of Hkv");
  if (a->Hq / a->Hkv > 16) return fail(KVSEL_E_UNSUPPORTED, "query heads per KV head must be <= 16");
  if (a->block_size % 16 != 0) return fail(KVSEL_E_UNSUPPORTED, "block_size must be a multiple of 16");
  if (a->Hkv > 4096) return fail(KVSEL_E_UNSUPPORTED, "Hkv must be <= 4096");
  if (a->n_cap < 0 || a->n_cap > (int64_t(1) << 30)) return fail(KVSEL_E_ARG, "n_cap must be in [0, 2^30]");
  if (static_cast<int64_t>(a->Y) * a->block_size > kMaxN) return fail(KVSEL_E_ARG, "Y * block_size must be below 2^31");
  if (!(a->scale >= 0.f) || isinf(a->scale)) return fail(KVSEL_E_ARG, "scale must be finite and >= 0");
  if (a->req == nullptr && a->Ra > a->R) return fail(KVSEL_E_ARG, "Ra > R needs an explicit req list");
  if (a->Ra > 0 && a->n_cap > 0) {
    if (a->Y < 1) return fail(KVSEL_E_ARG, "Y must be >= 1");
    if (a->q == nullptr || a->lse == nullptr || a->k_pool == nullptr || a->block_table == nullptr ||
        a->n_ctx == nullptr || a->n_seen == nullptr || a->state == nullptr)
      return fail(KVSEL_E_ARG, "a pointer is NULL");
    if (!aligned16(a->q) || !aligned16(a->k_pool)) return fail(KVSEL_E_ARG, "q and k_pool must be 16-byte aligned");
    const uintptr_t mis = reinterpret_cast<uintptr_t>(a->lse) | reinterpret_cast<uintptr_t>(a->block_table) |
                          reinterpret_cast<uintptr_t>(a->n_ctx) | reinterpret_cast<uintptr_t>(a->n_seen) |
                          reinterpret_cast<uintptr_t>(a->state) | reinterpret_cast<uintptr_t>(a->req);
    if ((mis & 3u) != 0) return fail(KVSEL_E_ARG, "lse, state and int32 arrays must be 4-byte aligned");
  }
  p->Ra = a->Ra; p->R = a->R; p->L = a->L; p->Hq = a->Hq; p->Hkv = a->Hkv; p->D = a->D;
  p->G = a->Hq / a->Hkv; p->block_size = a->block_size; p->Y = a->Y;
  const float scale = (a->scale == 0.f) ? 1.0f / sqrtf(static_cast<float>(a->D)) : a->scale;
  p->scale2 = scale * 1.4426950408889634f;
  p->n_cap = a->n_cap; p->pool_blocks = a->pool_blocks;
  p->req = a->req; p->block_table = a->block_table; p->n_ctx = a->n_ctx; p->n_seen = a->n_seen;
  return KVSEL_OK;
}

kvsel_status kvsel_decode_score(const kvsel_decode_args* a, void* stream) {
  try {
    DecodeParams p;
    kvsel_status s = check_decode(a, &p);
    if (s != KVSEL_OK) return s;
    if (p.Ra == 0 || p.n_cap == 0) return KVSEL_OK;
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_mode() && a->req != nullptr) {
      std::vector<int32_t> req;
      if ((s = debug_fetch(a->req, static_cast<size_t>(a->Ra), &req, st)) != KVSEL_OK ||
          (s = debug_distinct(req, a->R, "req")) != KVSEL_OK)
        return s;
    }
    return finish(launch_decode_score(p, a->dtype, a->q, a->lse, a->k_pool, a->state, st), st, "decode score");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

// ------------------------------------------------------------------ keep score

static kvsel_status check_keep_score(const kvsel_keep_score_args* a, KeepScoreParams* p) {
  if (a == nullptr) return fail(KVSEL_E_ARG, "args is NULL");
  if (a->struct_size < sizeof(kvsel_keep_score_args)) return fail(KVSEL_E_ARG, "struct_size too small");
  if (a->Rc < 0 || a->R < 0 || a->Rc > 65535) return fail(KVSEL_E_ARG, "Rc must be in [0, 65535] and R >= 0");
  if (a->L < 1 || a->Hkv < 1) return fail(KVSEL_E_ARG, "L and Hkv must be >= 1");
  if (static_cast<int64_t>(a->L) * a->Hkv > kMaxN) return fail(KVSEL_E_ARG, "L * Hkv too large");
  if (a->n_cap < 0 || a->n_cap > kMaxN) return fail(KVSEL_E_ARG, "n_cap must be in [0, 2^31)");
  if (!(a->lam >= 0.f && a->lam <= 1.f)) return fail(KVSEL_E_ARG, "lambda must be in [0, 1]");
  if (!(a->top_p > 0.f && a->top_p <= 1.f)) return fail(KVSEL_E_ARG, "top_p must be in (0, 1]");
  if (a->req == nullptr && a->Rc > a->R) return fail(KVSEL_E_ARG, "Rc > R needs an explicit req list");
  if (a->Rc > 0 && a->n_cap > 0) {
    if (a->n_len == nullptr || a->state == nullptr || a->keep_score == nullptr)
      return fail(KVSEL_E_ARG, "a pointer is NULL");
    const uintptr_t mis = reinterpret_cast<uintptr_t>(a->req) | reinterpret_cast<uintptr_t>(a->n_len) |
                          reinterpret_cast<uintptr_t>(a->state) | reinterpret_cast<uintptr_t>(a->keep_score) |
                          reinterpret_cast<uintptr_t>(a->attn_score);
    if ((mis & 3u) != 0) return fail(KVSEL_E_ARG, "float and int32 arrays must be 4-byte aligned");
  }
  p->Rc = a->Rc; p->R = a->R; p->L = a->L; p->Hkv = a->Hkv; p->n_cap = a->n_cap;
  p->lambda = a->lam; p->top_p = a->top_p; p->req = a->req; p->n_len = a->n_len;
  return KVSEL_OK;
}

kvsel_status kvsel_keep_score_workspace(const kvsel_keep_score_args* a, size_t* bytes) {
  try {
    if (bytes == nullptr) return fail(KVSEL_E_ARG, "bytes is NULL");
    KeepScoreParams p;
    kvsel_status s = check_keep_score(a, &p);
    if (s != KVSEL_OK) return s;
    *bytes = keep_score_workspace_bytes(p, a->attn_score != nullptr);
    return KVSEL_OK;
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}

kvsel_status kvsel_keep_score(const kvsel_keep_score_args* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    KeepScoreParams p;
    kvsel_status s = check_keep_score(a, &p);
    if (s != KVSEL_OK) return s;
    if (p.Rc == 0 || p.n_cap == 0) return KVSEL_OK;
    const size_t need = keep_score_workspace_bytes(p, a->attn_score != nullptr);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
      return fail(KVSEL_E_WORKSPACE, "workspace too small (see kvsel_keep_score_workspace)");
    if (need > 0 && !aligned16(ws)) return fail(KVSEL_E_ARG, "workspace must be 16-byte aligned");
    if ((s = check_device()) != KVSEL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_mode() && a->req != nullptr) {
      std::vector<int32_t> req;
      if ((s = debug_fetch(a->req, static_cast<size_t>(a->Rc), &req, st)) != KVSEL_OK ||
          (s = debug_distinct(req, a->R, "req")) != KVSEL_OK)
        return s;
    }
    return finish(launch_keep_score(p, a->state, a->keep_score, a->attn_score, a->hit, ws, st), st, "keep score");
  } catch (...) {
    return fail(KVSEL_E_ARG, "internal error");
  }
}
