/*
 * kvsel.h -- C ABI of libkvsel: attention-score-driven KV-cache selection on
 * AMD MI355X (gfx950).
 *
 * The three steps follow the workflow ActKV §3.3 (three primitives) describes:
 * attention calculation (kvsel_score), entry eviction to a keep mask
 * (kvsel_select), and materialisation of the kept set -- either a compact
 * re-RoPEd view (kvsel_gather_rerope, KVMem "tiered movement") or a slot-map
 * redirect to a dead slot with survivors left in place (kvsel_redirect,
 * IntentKV §2 Q2 and §4 "redirect").  kvsel_memory_update maintains the
 * session query memory that IntentKV §4 scores against.  For ActKV's own
 * policy, kvsel_decode_score keeps a running mean of recovered attention
 * over each action region (§7.1, Algorithm 3), kvsel_keep_score turns it
 * into LRFU keep scores at a compression step (§5.2), and kvsel_compact
 * compacts the pool in place after eviction (§7.2).  kvsel_free_list and
 * kvsel_build_index serve the redirect and block-scoring paths.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Plain C types only.  Every args struct begins with `struct_size`
 *   (set it to sizeof(the struct)) so the ABI can grow.
 * - Ownership: the caller allocates every buffer (device memory unless
 *   stated) and keeps it alive until the stream reaches the call.  The
 *   library allocates no device memory; scratch comes from the caller's
 *   workspace, sized by the *_workspace queries.  Outputs must not alias
 *   inputs except where an argument is documented "in/out".
 * - Execution: each call validates its arguments on the host, then enqueues
 *   kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *   returns without synchronising.  Results are valid once the stream
 *   reaches that point.  With the environment variable KVSEL_DEBUG=1 each
 *   call synchronises its stream and reports kernel errors, and NaN or Inf
 *   in the scores kvsel_select reads or kvsel_score writes is reported as
 *   E_ARG (for kvsel_score the outputs have then been written).  Debug mode
 *   also checks on the host the index lists in-place calls rely on
 *   (ascending block lists and distinct pages of an incremental view,
 *   blocks not shared between requests in a compaction, requests listed
 *   once for the ActKV calls) and reports violations as E_ARG.
 * - Errors: on any status other than KVSEL_OK nothing was enqueued and
 *   kvsel_last_error() describes why.  No C++ exception crosses the ABI.
 * - Device pointers must be 16-byte aligned; sizes are element counts.
 *   Inputs must be finite (NaN/Inf scores are outside the contract).
 * - Layouts are row-major, last index fastest.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVSEL_ABI_VERSION 1

typedef enum kvsel_status {
  KVSEL_OK = 0,
  KVSEL_E_ARG = 1,         /* null pointer, bad shape/enum, misalignment, N >= 2^31 */
  KVSEL_E_BUDGET = 2,      /* n_sink + n_recent > k_total while k_total < N */
  KVSEL_E_UNSUPPORTED = 3, /* dtype/shape combination not built, device is not gfx950 */
  KVSEL_E_WORKSPACE = 4,   /* workspace missing or smaller than the query returned */
  KVSEL_E_DEVICE = 5       /* a HIP call failed; the message carries hipGetErrorString */
} kvsel_status;

typedef enum kvsel_dtype { KVSEL_F32 = 0, KVSEL_BF16 = 1, KVSEL_F16 = 2 } kvsel_dtype;

typedef enum kvsel_score_mode {
  KVSEL_SCORE_WINDOW = 0, /* token level: softmax of a query window against every key */
  KVSEL_SCORE_MEMORY = 1, /* token level: softmax of the session memory row over history */
  KVSEL_SCORE_BLOCK = 2   /* block level: dot product with a RoPE-stripped Mean-K index */
} kvsel_score_mode;

typedef enum kvsel_agg { KVSEL_AGG_SUM = 0, KVSEL_AGG_MEAN = 1, KVSEL_AGG_MAX = 2 } kvsel_agg;
typedef enum kvsel_pool { KVSEL_POOL_NONE = 0, KVSEL_POOL_AVG = 1, KVSEL_POOL_MAX = 2 } kvsel_pool;
typedef enum kvsel_reduce { KVSEL_REDUCE_PER_UNIT = 0, KVSEL_REDUCE_GLOBAL = 1 } kvsel_reduce;
typedef enum kvsel_rope { KVSEL_ROPE_NONE = 0, KVSEL_ROPE_RAW = 1, KVSEL_ROPE_DELTA = 2 } kvsel_rope;
typedef enum kvsel_rope_style { KVSEL_ROPE_HALF = 0, KVSEL_ROPE_INTERLEAVED = 1 } kvsel_rope_style;
typedef enum kvsel_gather_mode { KVSEL_GATHER_FRESH = 0, KVSEL_GATHER_INCREMENTAL = 1 } kvsel_gather_mode;

/* ABI version of the loaded library (KVSEL_ABI_VERSION it was built with). */
int32_t kvsel_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next kvsel_* call on that thread. */
const char* kvsel_last_error(void);

/* ------------------------------------------------------------------ score
 *
 * Window mode -- ActKV §2 (attention score of a cached key = its softmax
 * weight) and §7.1 (probabilities recovered as exp(s - LSE) from the
 * log-sum-exp an attention pass already produced):
 *   s[r,j] = scale * q_r . k_j, rows r = (query head h of KV group g, window
 *   row t).  Window row t sits at position N-W+t; with `causal` it sees keys
 *   j <= N-W+t.  p = exp(s - LSE_r), LSE from `lse_in` if given, else
 *   computed (and written to `lse_out` if given; with `scores` NULL and
 *   `lse_out` given, the call computes only the LSE).  Per unit u = (l, g):
 *   a[u,j] = row_agg over t of (head_agg over h in g of p), then 1-D pooling.
 *   q: [L][Hq][W][D] (F32/BF16/F16, post-RoPE); k: [L][Hkv][N][D] (same
 *   dtype); lse_in/lse_out: [L][Hq][W] F32.  Output `scores`: [L*Hkv][N] F32.
 *
 * Memory mode -- IntentKV §4 (rule score): for every layer l and query head h,
 *   a[l,h,j] = softmax over the history H of scale * M[l,h] . K[l,g(h),j];
 *   H = positions that are neither forced (j < n_sink, j >= N - n_recent)
 *   nor redirected to the dead slot (slot_map[j] == dead_slot, IntentKV §3
 *   one-way eviction).  reduce GLOBAL: rule_j = sum over (l,h), summed in a
 *   fixed order (deterministic); PER_UNIT: sum over h in g per (l,g).
 *   q = M: [L][Hq][D] F32.  k = paged pool [L][pool_pages][page_size][Hkv][D]
 *   (BF16/F16), logical page p at physical page page_table[p] (ActKV §2
 *   paging).  Positions outside H score 0.  Output [N] (GLOBAL) or
 *   [L*Hkv][N] (PER_UNIT), F32.  page_size in [1, 64] with
 *   2 * page_size * Hkv * (2 * D + 16) <= 160 KiB (E_UNSUPPORTED beyond).
 *
 * Block mode -- KVMem (query-conditioned retrieval): per unit u = (l, g),
 *   q-bar[s,u] = sum over the W query tokens and the group's heads of the
 *   pre-RoPE query, and s[s,u,b] = scale * q-bar[s,u] . mu[u,b] against the
 *   F16 RoPE-stripped Mean-K index mu: [L][Hkv][N][D] (N = blocks per unit).
 *   Only index columns [n_begin, n_begin + n_count) are scored (bounded
 *   tiles).  q: [S][L][Hq][W][D] (BF16/F16/F32).  q-bar is computed into
 *   `qbar` ([S][L][Hkv][D] F32, or the workspace when NULL); with
 *   `qbar_valid` = 1 the call reads `qbar` instead and `q` may be NULL.
 *   Output `scores`: [S][L*Hkv][n_count] F32.
 *   Packed output (D = 128; `admit` and `tile_mask` both given, or both
 *   NULL for the dense output above): for tiled selection, where only
 *   columns above the running set's smallest score can still be selected.
 *   admit: [S][L*Hkv] F32, the thresholds a tiled kvsel_select call wrote
 *   (NaN admits every column).  Column b of a row is admitted when its
 *   score is greater than the row's threshold (-0.0 equals +0.0).  Each
 *   row is cut into chunks of 256 columns: chunk c stores the scores of its
 *   admitted columns, in ascending column order, at row positions
 *   [256 c, 256 c + admitted); the other positions are left unwritten.
 *   tile_mask: [S][L*Hkv][ceil(n_count / 64)] uint64, bit i of word w set
 *   when column 64 w + i is admitted.  kvsel_select reads this form when
 *   given the same tile_mask.
 *
 * Limits: L * Hkv <= 65535 (E_UNSUPPORTED beyond).
 * scale = 0 means 1/sqrt(D).  Pooling (window/memory-per-unit): centred,
 * odd `pool_k`, stride 1; AVG divides by pool_k counting out-of-range terms
 * as zero, MAX takes the in-range maximum.
 */
typedef struct kvsel_score_args {
  uint32_t struct_size;
  int32_t mode;         /* kvsel_score_mode */
  int32_t q_dtype;      /* kvsel_dtype of q */
  int32_t k_dtype;      /* kvsel_dtype of k / pool / index */
  int32_t L, Hq, Hkv, D;/* layers, query heads, KV heads, head dim (64 or 128) */
  int32_t W;            /* window rows (window) or query tokens per head (block) */
  int32_t S;            /* sessions (block mode); 1 otherwise */
  int64_t N;            /* cached positions (window/memory) or index blocks per unit (block) */
  const void* q;
  const void* k;
  /* memory mode: paging and history */
  const int32_t* page_table; /* [ceil(N/page_size)] logical page -> physical page */
  int32_t page_size;
  int32_t n_sink, n_recent;  /* forced set excluded from the history */
  int64_t pool_pages;        /* physical pages per layer in the pool */
  const int32_t* slot_map;   /* [N] or NULL: positions equal to dead_slot are dead */
  int64_t dead_slot;
  /* block mode: tile and query reduction */
  int64_t n_begin, n_count;
  float* qbar;
  int32_t qbar_valid;
  /* window mode */
  int32_t causal;
  const float* lse_in;  /* nullable */
  float* lse_out;       /* nullable */
  int32_t head_agg, row_agg; /* kvsel_agg */
  int32_t reduce;       /* kvsel_reduce (memory mode) */
  int32_t pool, pool_k; /* kvsel_pool, odd kernel size */
  float scale;
  float* scores;        /* output, F32 */
  /* block mode, packed output (struct_size ending before admit: dense) */
  const float* admit;   /* [S][L*Hkv] F32 thresholds, or NULL */
  uint64_t* tile_mask;  /* [S][L*Hkv][ceil(n_count / 64)] admission masks, or NULL */
} kvsel_score_args;

/* Bytes of device workspace kvsel_score needs for `args` (may be 0).
 * Memory mode keeps a float32 logit scratch of whole layers (Hq * N * 4
 * bytes per layer) at the end of its workspace and runs its logits -> LSE ->
 * rule kernels in passes over as many layers as that scratch holds: the
 * query asks for up to 512 MiB of scratch; a workspace shorter by whole
 * layers is accepted down to one layer of scratch (more passes, the same
 * results), and a shorter one fails with KVSEL_E_WORKSPACE. */
kvsel_status kvsel_score_workspace(const kvsel_score_args* args, size_t* bytes);

kvsel_status kvsel_score(const kvsel_score_args* args, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ select
 *
 * Budgeted top-k with a forced set -- IntentKV §4 (top-k selection: the
 * forced set plus the highest-scoring rest of the budget), KVMem
 * (query-conditioned retrieval: sink and recent always kept, the rest by
 * score, restored to chronological order), ActKV §3.3 (entry eviction
 * yields a Boolean keep mask).
 *
 * Per unit: F = [0, n_sink) U [n_total - n_recent, n_total); alive A = all
 * positions, or those with slot_map[j] != dead_slot.  The kept set is
 * (F n A) plus the k_total - |F n A| best positions of A \ F, ordered by
 * score descending with ties to the lower index (-0.0 equals +0.0); if
 * |A| <= k_total every alive position is kept.  Output in ascending order.
 *
 * scores: [U] rows of `n` F32 values, row u at scores + u*row_stride,
 * holding positions [base, base + n) of each unit.  One call with base = 0
 * and n = n_total selects directly.  Tiled use (KVMem scores its index in
 * bounded tiles): call once per tile in ascending `base`, passing running
 * candidate buffers cand_score/cand_idx ([U][k_total] each) and cand_count
 * ([U], zeroed by the caller before the first tile); the last tile sets
 * `finalize` = 1.  The tiled result equals the untiled one.
 * Admission (tiled calls): a call that does not finalize writes, with
 * `admit` given ([U] F32), the score no later column can tie or beat and
 * still enter: the running set's smallest score once it holds every slot
 * left beside the forced set, NaN before.  Scored with that threshold
 * (kvsel_score block mode, packed output), the next tile is passed as its
 * packed scores plus `tile_mask` ([U][ceil(n / 64)] uint64, the same
 * layout); the result equals the dense tile's.  Thresholds that are not
 * above the previous call's `admit` (NaN included) keep that equality;
 * higher ones may drop columns that belong to the result.
 * Outputs (written when finalize = 1, or on an untiled call): kept_idx
 * [U][k_total] int32 ascending, -1 past n_kept; n_kept [U] (nullable);
 * keep_mask [U][n_total] u8 (nullable; untiled calls only).
 * Optional pooling (untiled calls only): with pool != KVSEL_POOL_NONE the
 * selection ranks pool(scores) instead of the scores themselves, the same
 * centred 1-D pooling kvsel_score offers (odd pool_k; AVG counts
 * out-of-range terms as zero, MAX takes the in-range maximum), computed on
 * the fly while the keys are formed.
 * Workspace: kvsel_select_workspace() bytes, 16-byte aligned (the ordering
 * key of every position of the call, small per-slice histograms, and for at
 * most 8 units of rows longer than 32768 positions a few more per-slice
 * histograms and counts: about 4 bytes per position); 0 when U or n is 0, and for untiled calls without a
 * slot map, unpooled or MAX-pooled with pool_k <= 9 (AVG-pooled with pool_k
 * <= 9 too when n <= 2048), over at least 128 units of at most 32768
 * positions, or over any number of units of at most 8192 positions, whose
 * per-unit workgroups keep their keys in registers.
 * Errors: KVSEL_E_BUDGET if n_sink + n_recent > k_total and k_total < n_total;
 * KVSEL_E_WORKSPACE if the workspace is missing or too small; KVSEL_E_UNSUPPORTED
 * for U > 65535, and for `tile_mask` or `admit` on a tiled call that needs
 * the workspace (k_total above 8192, or tiles too wide for one workgroup's
 * LDS); KVSEL_E_ARG for `tile_mask` or `admit` on an untiled call.
 */
typedef struct kvsel_select_args {
  uint32_t struct_size;
  int32_t U;
  int64_t n;
  int64_t row_stride;
  const float* scores;
  int64_t base;
  int64_t n_total;
  int32_t k_total, n_sink, n_recent;
  const int32_t* slot_map;   /* [n_total] or NULL, shared by all units */
  int64_t dead_slot;
  float* cand_score;         /* [U][k_total] or NULL (tiled use) */
  int32_t* cand_idx;         /* [U][k_total] or NULL */
  int32_t* cand_count;       /* [U] or NULL */
  int32_t finalize;
  int32_t* kept_idx;         /* [U][k_total] */
  uint8_t* keep_mask;        /* [U][n_total] or NULL */
  int32_t* n_kept;           /* [U] or NULL */
  int32_t pool, pool_k;      /* kvsel_pool and odd kernel size (untiled calls) */
  /* tiled calls (struct_size ending before tile_mask: dense tiles, no admission output) */
  const uint64_t* tile_mask; /* [U][ceil(n / 64)]: the tile is packed; NULL: dense */
  float* admit;              /* [U] F32, written by calls that do not finalize; or NULL */
} kvsel_select_args;

kvsel_status kvsel_select_workspace(const kvsel_select_args* args, size_t* bytes);

kvsel_status kvsel_select(const kvsel_select_args* args, void* workspace,
                          size_t workspace_bytes, void* stream);

/* kvsel_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, validation and results
 * as kvsel_select; the scratch kvsel_select_workspace() would report lives
 * instead in a fixed array of KVSEL_NOALLOC_SCRATCH_BYTES per device inside
 * the library, reserved on each GPU the library runs on until the process
 * ends.  The call itself allocates nothing.
 * Sharing: every call on one GPU uses that GPU's array, so calls that
 * overlap on one GPU (different streams, or host threads racing on one
 * device) race and give undefined results; serialise them.  Each call writes
 * every scratch word it reads, so no state carries over between calls.
 * Errors: as kvsel_select, plus KVSEL_E_WORKSPACE when
 * kvsel_select_workspace() would exceed KVSEL_NOALLOC_SCRATCH_BYTES (about
 * 4 bytes per score of an untiled call; tiled calls need none), and
 * KVSEL_E_DEVICE if the array's device address cannot be resolved. */
#define KVSEL_NOALLOC_SCRATCH_BYTES (64u << 20)

kvsel_status kvsel_select_noalloc(const kvsel_select_args* args, void* stream);

/* ------------------------------------------------------------------ gather
 *
 * Materialise a selection as a compact view -- KVMem (tiered movement):
 * kept blocks are packed into contiguous logical positions; K is rotated
 * for the new position and V is copied as is.
 *
 * FRESH: for unit u and kept entry i (ascending), rows o < bt:
 *   dst[u][i*bt + o] = R(p) src[u][idx[u][i]*bt + o], with
 *   rope NONE: no rotation (bitwise copy); RAW: p = pos0 + i*bt + o (raw,
 *   position-free K); DELTA: p = (pos0 + i*bt + o) - (idx*bt + o) (K already
 *   rotated at its old position).  V is always copied bitwise.
 *   Rotation: rotate-half (pairs m, m + rotary_dim/2) or interleaved (pairs
 *   2m, 2m+1), inv_freq[m] = theta^(-2m/rotary_dim); angles are formed in
 *   float64.  src of unit u starts at src_k + src_offsets[u] elements
 *   (src_offsets: device int64 [U], or NULL for u * src_unit_stride), so
 *   several units may alias one buffer.  dst: [U][k*bt][D].
 *   Entries with i >= n_idx[u] (when n_idx is given) are left untouched.
 *
 * INCREMENTAL (reuse of overlapping pages across steps): per unit the
 *   previous view holds blocks prev_idx[u][:k] (ascending) in pages
 *   prev_page[u][:k] of a pool [U][pool_pages][bt][D] (pool_k/pool_v, in/out).
 *   A block in both views keeps its page and V; when its position moved its
 *   K is rotated in place by (i_new - i_old)*bt (hit_raw = 0: the GPU copy
 *   alone suffices, but each move adds one bf16 rounding to that block's K),
 *   or, with hit_raw = 1, replaced by its raw K from src_k rotated to
 *   pos0 + i_new*bt + o (one rounding, whatever the number of moves; needs
 *   src_k, read by block id like a miss).  Pages of blocks that left
 *   the view are taken in ascending page order by the new blocks in
 *   ascending block order; those get K = R(pos0 + i_new*bt + o) raw K and
 *   V copied, both read from src (as in FRESH), or, when staged_k is given,
 *   from packed staging buffers: the i-th miss of unit u (misses in
 *   ascending block order) at entry i of staged_k/staged_v
 *   [U][staged_cap][bt][D] (the state after KVMem's host gather and
 *   host-to-device copy of the missed blocks); src_k/src_v may then be NULL.
 *   Misses of rank >= staged_cap are skipped (their pages keep their bytes).
 *   Out: page_table [U][k] (page of each kept block, chronological),
 *   n_miss [U].  idx holds the new selection [U][k] (ascending, all valid).
 * Workspace: INCREMENTAL needs kvsel_gather_workspace() bytes (4 per entry:
 *   the plan that pairs every new entry with its previous position or its
 *   miss rank, written by one launch and read by the next); FRESH needs none.
 *   The call takes a workspace so that it allocates nothing itself.
 * ABI: staged_k, staged_v, staged_cap and hit_raw were appended to the
 *   struct; a caller whose struct_size ends before them gets the raw-source
 *   form with hits rotated in place.
 */
typedef struct kvsel_gather_args {
  uint32_t struct_size;
  int32_t mode;          /* kvsel_gather_mode */
  int32_t U, D;
  int32_t dtype;         /* kvsel_dtype of K/V (BF16, F16 or F32) */
  int32_t bt;            /* rows per selected entry (1 = tokens, 32 = blocks) */
  int32_t k;             /* entries per unit */
  const void* src_k;
  const void* src_v;
  const int64_t* src_offsets; /* device [U] element offsets, or NULL */
  int64_t src_unit_stride;    /* elements, used when src_offsets is NULL */
  int64_t src_rows;           /* rows available per unit source (bounds check) */
  const int32_t* idx;         /* [U][k] */
  const int32_t* n_idx;       /* [U] or NULL (FRESH only) */
  void* dst_k;                /* FRESH: [U][k*bt][D] */
  void* dst_v;
  int32_t rope;               /* kvsel_rope */
  int32_t style;              /* kvsel_rope_style */
  int32_t rotary_dim;         /* 0 = D */
  double theta;
  int64_t pos0;
  /* INCREMENTAL */
  const int32_t* prev_idx;    /* [U][k] */
  const int32_t* prev_page;   /* [U][k] */
  void* pool_k;               /* [U][pool_pages][bt][D], in/out */
  void* pool_v;
  int64_t pool_pages;
  int32_t* page_table;        /* out [U][k] */
  int32_t* n_miss;            /* out [U] */
  /* INCREMENTAL, optional: packed misses */
  const void* staged_k;       /* [U][staged_cap][bt][D] or NULL (misses from src) */
  const void* staged_v;
  int64_t staged_cap;         /* entries per unit in the staging buffers */
  int32_t hit_raw;            /* INCREMENTAL: 1 = moved hits re-rotated from src_k */
  int32_t reserved;           /* 0 */
} kvsel_gather_args;

kvsel_status kvsel_gather_workspace(const kvsel_gather_args* args, size_t* bytes);

kvsel_status kvsel_gather_rerope(const kvsel_gather_args* args, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ redirect
 *
 * IntentKV §4 (redirect) and §2 Q2: every dropped logical position is
 * pointed at one sentinel dead slot; kept positions keep their slot ids and
 * nothing moves.  slot_map [N] int32 in/out; keep_mask [N] u8 (1 = keep),
 * or, when keep_mask is NULL, the kept positions themselves: kept_idx [k]
 * int32 in ascending order, entries < 0 ignored (the -1 tail kvsel_select
 * writes past n_kept), entries >= N never match; k = 0 keeps nothing
 * (kept_idx may then be NULL).  Already-dead entries stay dead.
 * (struct_size ending before kept_idx: the keep_mask form only.)
 * Sentinel init (optional, when k_pool is non-NULL): writes the dead slot's
 * rows in every layer and KV head: K = -1e4 rounded to the pool dtype
 * (bf16 -9984, f16 -10000), V = 0.  Pools are [L][pool_slots][Hkv][D] with
 * pool_slots = pool_pages * page_size, i.e. the paged layout flattened.
 */
typedef struct kvsel_redirect_args {
  uint32_t struct_size;
  int64_t N;
  int32_t* slot_map;
  const uint8_t* keep_mask;
  int64_t dead_slot;
  void* k_pool;          /* nullable: skip the sentinel write */
  void* v_pool;
  int32_t L, Hkv, D;
  int32_t dtype;         /* BF16 or F16 */
  int64_t pool_slots;    /* slots per layer */
  const int32_t* kept_idx; /* [k] ascending, or NULL (keep_mask form) */
  int32_t k;
} kvsel_redirect_args;

kvsel_status kvsel_redirect(const kvsel_redirect_args* args, void* stream);

/* ------------------------------------------------------------------ free list
 *
 * IntentKV §7 (alias-aware deallocation) and §4 minimum check 6: after a
 * compression step, the physical slot u = slot_map[j] of a dropped position
 * j may go back to the allocator only if (a) j >= protected_len (outside the
 * radix-protected prefix), (b) u != dead_slot, and (c) no kept position
 * maps to u (this catches slots shared by aliases).  Call it with the slot
 * map as it was BEFORE kvsel_redirect overwrites the dropped positions.
 *
 *   slot_map    [N] int32 (not modified); keep_mask [N] u8 (1 = kept)
 *   n_slots     physical slot ids lie in [0, n_slots); ids outside are never
 *               freed (nor the dead slot)
 *   free_slots  out [N] int32: the distinct freed slots in ascending order,
 *               then -1 up to N
 *   n_free      out [1] int32: how many were freed
 * Workspace: kvsel_free_list_workspace (two bitmaps over the slot ids).
 * Errors: E_ARG (NULL pointers, N outside [0, 2^31), n_slots outside
 * [1, 2^31), protected_len < 0, pointers not 4-byte aligned),
 * E_WORKSPACE, E_DEVICE.  N = 0 writes n_free = 0.
 */
typedef struct kvsel_freelist_args {
  uint32_t struct_size;
  int32_t reserved;          /* 0 */
  int64_t N;
  const int32_t* slot_map;
  const uint8_t* keep_mask;
  int64_t dead_slot;
  int64_t protected_len;
  int64_t n_slots;
  int32_t* free_slots;
  int32_t* n_free;
} kvsel_freelist_args;

kvsel_status kvsel_free_list_workspace(const kvsel_freelist_args* args, size_t* bytes);

kvsel_status kvsel_free_list(const kvsel_freelist_args* args, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------ compaction
 *
 * ActKV §7.2 (conflict-free slot planning) and Algorithm 4 (in-place
 * compaction): after eviction, each request's kept entries move into its last
 * X = ceil(kept / block_size) logical blocks, and the blocks before them are
 * returned.  Slots are planned first: the i-th kept position before the
 * target region (ascending) goes to the i-th slot of the region that holds
 * no kept entry (ascending; slots past N count as empty).  Sources and
 * destinations are disjoint physical slots, so every copy runs in one pass
 * with no buffer for KV.  (The page's formula for the region is lost; this is
 * the reading used.)
 *
 *   keep_mask    [R][N] u8 (1 = kept)
 *   block_table  [R][Y] int32: physical block of each logical block; a
 *                request's blocks must be distinct and not shared with other
 *                requests (entries outside [0, pool_blocks) are not copied)
 *   k_pool/v_pool [L][pool_blocks][block_size][Hkv][D] of dtype, in place
 *   slot_pos     out [R][Y * block_size] int32: the original logical position
 *                each slot holds afterwards, -1 for empty slots and for the
 *                freed blocks
 *   freed_blocks out [R][Y] int32: physical blocks of logical blocks
 *                [0, Y - X) in order, then -1; n_freed out [R] = Y - X
 * Requirements: 0 <= N <= Y * block_size, Hkv * D * element size a multiple
 * of 16 bytes, pools 16-byte aligned.  Workspace: kvsel_compact_workspace.
 * Errors: E_ARG, E_WORKSPACE, E_UNSUPPORTED (R > 65535), E_DEVICE.  R = 0 or Y = 0 is a
 * no-op.
 */
typedef struct kvsel_compact_args {
  uint32_t struct_size;
  int32_t R;
  int32_t L, Hkv, D;
  int32_t dtype;              /* BF16, F16 or F32 */
  int32_t block_size;
  int32_t Y;                  /* logical blocks per request */
  int32_t reserved;           /* 0 */
  int64_t N;                  /* positions per request */
  int64_t pool_blocks;        /* physical blocks per layer */
  const uint8_t* keep_mask;
  const int32_t* block_table;
  void* k_pool;
  void* v_pool;
  int32_t* slot_pos;
  int32_t* freed_blocks;
  int32_t* n_freed;
} kvsel_compact_args;

kvsel_status kvsel_compact_workspace(const kvsel_compact_args* args, size_t* bytes);

kvsel_status kvsel_compact(const kvsel_compact_args* args, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------ index
 *
 * KVMem (query-conditioned retrieval paragraph): the block scorer reads one
 * RoPE-stripped mean key per (layer, KV head, bt-token block), kept in HBM as
 * an fp16 index that grows as blocks fill.  kvsel_build_index writes
 *   mu[u][b][:] = fp16_rne( (1/bt) * sum over the bt raw rows of block b )
 * for blocks b in [b_begin, b_begin + b_count) of every unit u.  The sum is
 * taken in float64 and rounded once to fp16 (round to nearest even), so the
 * index is bit-exact whenever the float64 sum of a block is exact (any block
 * whose raw values span fewer than 2^45 in magnitude).
 *
 *   src_k       raw (pre-RoPE) keys of unit u at src_k + offset(u) elements,
 *               rows [src_rows][D] of `dtype` (BF16, F16 or F32);
 *               offset(u) = src_offsets[u] (device int64 [U]) if given, else
 *               u * src_unit_stride (units may alias one buffer)
 *   mu          out: F16 [U][NB][D]; only the requested blocks are written
 *   D           64 or 128; bt in [1, 256]; 0 <= b_begin, b_count >= 0,
 *               b_begin + b_count <= NB and (b_begin + b_count) * bt <= src_rows
 * Errors: E_ARG (NULL pointers, ranges, alignment of src_k/mu to 16 bytes,
 * bad dtype), E_UNSUPPORTED (D), E_DEVICE.  b_count = 0 or U = 0 is a no-op.
 */
typedef struct kvsel_index_args {
  uint32_t struct_size;
  int32_t U, D;
  int32_t dtype;              /* kvsel_dtype of the raw keys */
  int32_t bt;                 /* rows per block (32 in KVMem) */
  const void* src_k;
  const int64_t* src_offsets; /* device [U] element offsets, or NULL */
  int64_t src_unit_stride;    /* elements, used when src_offsets is NULL */
  int64_t src_rows;           /* rows available per unit */
  int64_t NB;                 /* blocks per unit in mu */
  int64_t b_begin, b_count;   /* block range to (re)build */
  uint16_t* mu;               /* out: fp16 bit patterns [U][NB][D] */
} kvsel_index_args;

kvsel_status kvsel_build_index(const kvsel_index_args* args, void* stream);

/* ------------------------------------------------------------------ decode scorer
 *
 * ActKV §7.1 and Algorithm 3 (recovery-based attention calculation): for the
 * current query token of each request that is generating an action, every
 * cached key j of KV head g gets
 *   p[j] = max over the group's query heads h of exp(scale * q_h . k_j - LSE_h)
 * with LSE_h the natural-log log-sum-exp the paged attention pass produced
 * for that token and head, and p is folded into a running mean over the
 * action tokens of the current region:
 *   t = n_seen[r];  state <- (t == 0) ? p : state + (p - state) / (t + 1).
 * Keys come straight from the paged pool through the block table (ActKV §2
 * paging); nothing is gathered.  Readings where the page is silent: the
 * token sees the first n_ctx[r] positions; a position it cannot see, or
 * whose block-table entry lies outside [0, pool_blocks), has p = 0.
 *
 *   req          [Ra] int32 request (row of block_table, n_ctx, n_seen, state)
 *                of each query row, or NULL for rows 0..Ra-1 (then Ra <= R);
 *                entries outside [0, R) are skipped; a request may appear once
 *   q            [L][Ra][Hq][D] of dtype (BF16 or F16), post-RoPE
 *   lse          [L][Ra][Hq] F32, natural log
 *   k_pool       [L][pool_blocks][block_size][Hkv][D] of dtype
 *   block_table  [R][Y] int32
 *   n_ctx        [R] int32, clamped to [0, min(n_cap, Y * block_size)]
 *   n_seen       [R] int32, action tokens of the region already in the state
 *                (0 = this token starts a region; negative counts as 0)
 *   state        [L][R][Hkv][n_cap] F32, in/out
 * At t = 0 every position [0, n_cap) of the request is written (p, or 0
 * past n_ctx).  At t > 0 only positions in the 64-aligned tiles that hold
 * visible keys are written; positions past n_ctx must then hold 0, as a
 * region start leaves them (n_ctx does not decrease within a region), and
 * the state equals the plain mean over the region's tokens.
 * Requirements: D 64 or 128; G = Hq / Hkv integral and <= 16; block_size a
 * multiple of 16; Hkv <= 4096; Ra and L <= 65535; n_cap <= 2^30; q, k_pool
 * 16-byte aligned.  scale = 0 means 1/sqrt(D).
 * Errors: E_ARG (sizes, pointers, alignment), E_UNSUPPORTED (D, dtype,
 * G > 16, block_size, Hkv > 4096), E_DEVICE.  Ra = 0 is a no-op.
 */
typedef struct kvsel_decode_args {
  uint32_t struct_size;
  int32_t Ra, R;
  int32_t L, Hq, Hkv, D;
  int32_t dtype;              /* BF16 or F16 */
  int32_t block_size;
  int32_t Y;                  /* block-table columns per request */
  float scale;                /* 0 = 1/sqrt(D) */
  int64_t n_cap;              /* state positions per (layer, request, KV head) */
  int64_t pool_blocks;
  const int32_t* req;
  const void* q;
  const float* lse;
  const void* k_pool;
  const int32_t* block_table;
  const int32_t* n_ctx;
  const int32_t* n_seen;
  float* state;
} kvsel_decode_args;

kvsel_status kvsel_decode_score(const kvsel_decode_args* args, void* stream);

/* ------------------------------------------------------------------ keep score
 *
 * ActKV §5.2 (attention-aware LRFU) at a compression step, for the requests
 * in `req` (those that just left an action region):
 *   score[j] = float32( sum over layers l and KV heads g of state[l][r][g][j] )
 *              (summed in float64 with compensation, rounded once);
 *   hit[j]   = j is in the shortest prefix of the entries j < n_len[r], by
 *              score descending with the lower index first on ties, whose
 *              cumulative score reaches top_p * (sum of all scores); no hits
 *              when that product is 0;
 *   KS[j]    = lambda * KS[j] + (hit[j] ? score[j] : 0).
 * The page's update equation is lost; this is the reading whose limits are
 * the ones the page describes (lambda = 0: only the latest step counts;
 * lambda = 1: hits accumulate without decay).  Cumulative sums are float64;
 * where they fall within about 1e-15 of the target the boundary entry may
 * differ from an exact sequential sum's.
 *
 *   req         [Rc] int32, or NULL for 0..Rc-1 (then Rc <= R); entries
 *               outside [0, R) are skipped; a request may appear once
 *   n_len       [R] int32 entries per request, clamped to [0, n_cap]
 *   state       [L][R][Hkv][n_cap] F32 running means (kvsel_decode_score),
 *               non-negative
 *   keep_score  [R][n_cap] F32 in/out; entries j >= n_len keep their value
 *   attn_score  [R][n_cap] F32 out or NULL: score[j], 0 for j >= n_len
 *   hit         [R][n_cap] u8 out or NULL: 1 = hit (the entry's bit of the
 *               action access vector of ActKV §5.1 for this region), 0 for
 *               j >= n_len
 * lambda in [0, 1], top_p in (0, 1], Rc <= 65535, n_cap < 2^31.
 * Workspace: kvsel_keep_score_workspace (Rc * n_cap floats when attn_score
 * is NULL, else 0).
 * Errors: E_ARG, E_WORKSPACE, E_DEVICE.  Rc = 0 is a no-op.
 */
typedef struct kvsel_keep_score_args {
  uint32_t struct_size;
  int32_t Rc, R;
  int32_t L, Hkv;
  int32_t reserved;           /* 0 */
  int64_t n_cap;
  float lam;                  /* decay lambda in [0, 1] */
  float top_p;
  const int32_t* req;
  const int32_t* n_len;
  const float* state;
  float* keep_score;
  float* attn_score;
  uint8_t* hit;
} kvsel_keep_score_args;

kvsel_status kvsel_keep_score_workspace(const kvsel_keep_score_args* args, size_t* bytes);

kvsel_status kvsel_keep_score(const kvsel_keep_score_args* args, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------ memory
 *
 * IntentKV §4 (memory recurrence) and §7 (unit-norm projection): one turn
 *   M <- normalise(decay * M + mean over the turn's W query rows of q),
 * normalised to unit L2 norm along D per (layer, query head); a zero vector
 * stays zero.  q_turn: [L][Hq][W][D] (BF16/F16/F32); M: [L][Hq][D] F32 in/out.
 */
typedef struct kvsel_memupd_args {
  uint32_t struct_size;
  int32_t L, Hq, D, W;
  int32_t q_dtype;
  const void* q_turn;
  float* M;
  float decay;
} kvsel_memupd_args;

kvsel_status kvsel_memory_update(const kvsel_memupd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
