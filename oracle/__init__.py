"""Plain CPU fp64 oracle for the self-speculative decoding attention path.

This package is TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import it. The product (the HIP library and its
Python binding) never imports, calls or links anything from here, and nothing here
imports the product: the two share no code. Inputs reach both sides from the seeded
generator module, which holds none of the method's arithmetic.

Every function computes in numpy float64 and reads the exact stored input values
(bf16 bit patterns are widened exactly). Each module cites the passage of
"MagicDec: Breaking the Latency-Throughput Tradeoff for Long Context Generation with
Speculative Decoding" (arXiv 2408.11049v5) that it follows; where the paper is silent
the reading taken is stated in the docstring.

Modules
-------
kvcache    exact widening of stored values; paged-cache row gather, KV append, compact
           draft rows
attention  verify (gamma+1 causal queries), decode, sparse draft attention
streaming  StreamingLLM sink + recent-window draft set
snapkv     observation-window scoring, max-pool, per-KV-head top-k
philox     Philox4x32-10 counter-based generator and the uniform mapping
accept     greedy and rejection-sampling acceptance (Leviathan et al.)
topk       dynamic Top-K draft attention (per-step selection)
"""

from . import kvcache, attention, streaming, snapkv, philox, accept, topk  # noqa: F401
