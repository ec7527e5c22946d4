"""CPU oracle for softmax attention and its HyperAttention approximation.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code,
constants, tables or helpers with the HIP library under
``approximate_softmax_attention_amd/`` and never imports it.

Everything here is plain, slow and meant to be checked by eye against the
source pages. All floating-point arithmetic is fp64 (inputs given in fp32 or
bf16 are upcast exactly), except the rotary embedding, whose reading fixes
fp32 steps (rope.py states it and offers an fp64 adjoint); all index
arithmetic is exact integer arithmetic.

Sources
-------
"HA page": the Japanese article on HyperAttention at nearauto.com/p/20145.html
(title: a new approximate attention mechanism, HyperAttention, suited to long
contexts, making LLM inference 50% faster; it summarises arXiv 2310.05869).
Its sections are cited by their English gloss:

* "Method overview"  (dot-product attention, A, D, the softmax matrix,
  Eq. (1), sampling by the row norms of V, uniform sampling for D)
* "Algorithm"        (Definition 1 sortLSH, Algorithms 1-4, Figures 1-2)
* "Monkey-patching"  (recursion until n < 4096, b = m = 256)
* "Single self-attention layer" (split Q, K, V and merge outputs when causal)

The page lost its formulas, its pseudo-code and its figures in extraction.
Where a step is left open the module that implements it states the reading
it takes; the same list of readings is kept in the repository's design notes.

Modules
-------
rng            counter-based SplitMix64 draws (published generator)
exact          exact attention Att = D^-1 exp(QK^T) V, causal and not
sortlsh        hyperplanes, Hamming-sorted hash, sortLSH buckets
sampling       uniform column samples and V-row-norm samples
hyperattention ApproxD + HyperAttention (non-causal), causal recursion, merge
backward       gradients of exact attention and of the HyperAttention estimator
rope           rotary position embedding of Q and K before hashing, and its
               transpose (the gradient through it)
"""
