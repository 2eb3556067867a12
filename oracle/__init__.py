"""CPU oracle for the offloaded mixture-of-experts layer with an LRU expert cache.

TEST INFRASTRUCTURE ONLY.  A plain, slow, float64 NumPy implementation of
what the GPU library computes, written from the pages' description of the
method.  Only the test suite, the smoke entry point and the benchmark's CPU
baseline leg may import it; the library never does, and nothing here
imports the library.

Modules
-------
formats  decode tables for e2m1 and OCP E4M3, dequantisation of a packed
         expert block (int4 group-32 fp16 scale, e2m1 group-16 E4M3 scale, fp32)
route    router: logits, softmax, top-k with lowest-index tie-break
lru      two independent LRU slot-pool simulations (linked list, timestamps),
         wave split, a whole-run replay with statistics, prefill plan
ffn      SwiGLU expert FFN, the MoE layer, a dense brute-force variant
toy      the toy sticky router and per-pick LRU replay of the explainer page
report   bus / preflight arithmetic printed on the pages

Parity status: every function is pinned by a test under tests/ that does
not re-derive it from this code (worked examples, closed forms, a second
implementation or a library routine, printed values of the pages), except
where a function's header says "parity unpinned".
"""
