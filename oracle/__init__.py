"""Plain CPU oracle for attention-score-driven KV-cache selection.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The product path (``selection_score_amd`` and ``libkvsel.so``) never imports,
links or calls it, and it imports nothing from the product path.

Every function is a slow, direct transcription of what the pages define,
computed in float64 with NumPy.  Outputs that the GPU produces in float32 are
the float64 result rounded once (round-to-nearest-even); bfloat16/float16
outputs are the float64 result rounded once to that format
(``oracle.numerics``).  Library primitives (matmul, sort, exp, cos/sin) serve
as single steps; there is no blocking, fusion or reordering beyond what the
definitions state.

Sources (pages, by title and section):

* ActKV: Efficient LLM Agents through Action-Guided KV Cache Management --
  §2 (attention score and output; paged KV layout and the block-table
  example), §3.3 (the three primitives: attention calculation, entry
  eviction to a Boolean keep mask, cache compaction), §5.2 (the LRFU keep
  score with a top-p hit), §7.1 (recovering attention probabilities from
  the softmax log-sum-exp; Algorithm 3, the decode-streaming scorer).
* IntentKV: Cross-Turn Intent-Aware KV Cache Pruning for Agent Inference --
  §2 Q2 (retention/layout split, dead-slot sentinel), §3 (budget semantics,
  one-way eviction), §4 (top-k with forced set, memory recurrence, rule
  score, residual, redirect; minimum checks 1-3), §7 (unit-norm projection).
* KVMem: Virtualizing Million-Token Agent Workspaces on a Consumer GPU --
  the "query-conditioned retrieval" and "tiered movement" mechanisms
  (RoPE-stripped Mean-K block scoring; forced sink+recent blocks; fill by
  score; chronological restore; re-RoPE of raw K at new contiguous positions;
  V copied; overlapping pages kept).

Parity status per function is listed in ``PIN_STATUS`` below: "pinned" means
a ``-m "not gpu"`` test checks the function against something other than
itself (a worked example printed on the pages, a closed form, an invariant, a
textbook special case, or brute force on tiny inputs).
"""

PIN_STATUS = {
    "numerics.round_to_bf16/f16/f32": "pinned (bit patterns of known values, RNE halfway cases)",
    "paging.slot_map_from_block_table": "pinned (worked example of ActKV §2)",
    "score.window_scores": "pinned (hand-computed closed forms, causality, GQA map, row sums)",
    "score.pool1d": "pinned (impulse responses, coverage-count closed form)",
    "score.memory_update": "pinned (EMA closed forms, unit norm, fixed point)",
    "score.memory_scores": "pinned (cross-formulation with window_scores at W=1; sum = L*Hq)",
    "score.query_reduce / block_scores": "pinned (per-query brute force by linearity; hand example)",
    "score.mean_k_index": "pinned (hand-computed means over two blocks, fp16 RNE halfway cases, "
                          "constant blocks, linearity of the block score)",
    "score.decode_recovery_step": "pinned (running mean over T tokens equals the batch window mean "
                                  "with max over the group; LSE identity; hand two-token example; "
                                  "region reset)",
    "select.action_scores / top_p_hits": "pinned (hand-worked top-p sets, ties, top_p = 1; minimum "
                                         "cardinality by brute force over all subsets; exact unit sum)",
    "select.lrfu_keep_score": "partly unpinned: the page's update equation is lost; the reading "
                              "lam*KS + hit*score is pinned to the page's lambda = 0 (recency) and "
                              "lambda = 1 (frequency) limits, and for 0 < lambda < 1 only to the "
                              "behaviour the page describes (quiet intermittent entries survive, "
                              "stale continuous ones are overtaken), not to a formula",
    "score.residual_score": "pinned (zero-initialised fc2 gives the rule score exactly)",
    "select.select_topk": "pinned (exhaustive max-sum brute force on tiny inputs; invariants)",
    "select.select_topk_tiled": "pinned (equal to select_topk for every tile size)",
    "rope.rope_rotate": "pinned (D=2 textbook rotation, identity, norm, composition, relative property)",
    "materialise.gather_view": "pinned (bitwise element loops on tiny inputs; raw->baked identity)",
    "materialise.incremental_view": "pinned (equals a fresh build of the new selection; disjointness)",
    "materialise.redirect": "pinned (invariants: kept bitwise, dropped -> dead, idempotent, one-way)",
    "materialise.free_list": "pinned (hand-worked slot maps with aliases, prior redirects and a "
                             "protected prefix; reusing freed slots never changes a kept or sibling read)",
    "materialise.tail_compact": "pinned (hand-worked plan; kept (position, K, V) multiset preserved; "
                                "sources and destinations disjoint; freed count Y - X); the pairing "
                                "order is a reading (the page's formula is lost)",
    "materialise.decode_attention_*": "pinned (dead-slot closed form in both sign regimes)",
}
