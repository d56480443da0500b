"""CPU oracle for the tree-verification step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct restatement of what the step computes, used to
check the HIP library.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it; the library never does, and the two
share no code (the only thing both sides see is the seeded input generator).

Modules
  tree       -- draft-tree build (dynamic global top-k and static branching),
                ancestor mask / positions / retrieve paths, greedy acceptance
                (walk and the cumprod-over-paths formulation).
  attention  -- tree-masked GQA attention, dense softmax in float64.
  kv         -- compaction of the accepted path's K/V rows.
  sampling   -- target logits filtered into probabilities (temperature, top-k,
                top-p, min-p) and tree rejection sampling with the drafter's
                distribution q (min(1, p/q), residual norm(max(0, p - q))).

Sources (cited per function by page title and section):
  [HB]  AI-infra handbook, "Advanced speculative decoding: tree drafts and EAGLE"
        (tree_spec.py listing, correctness check, exercises).
  [E2]  EAGLE v2 dynamic-tree decoding walkthrough: sections 2 initialize_tree,
        3 topK_generate, 4 tree_decoding, 5 evaluate_posterior.
  [TRT] "TensorRT-LLM source dissection (22): EAGLE-3 one-model drafter", section
        "dynamic draft tree" (three ledgers: parents / packed mask / positions,
        tree-build kernel, greedy verification, KV relocation).

Parity pins: every function here is pinned by the non-GPU tests in tests/ against
values the pages print, closed forms, invariants, brute force on tiny inputs and
an independent library routine (torch SDPA) -- see each test module's header.
"""
