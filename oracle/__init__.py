"""Plain, slow, float64 CPU oracle for context-parallel attention shards.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only the test suite (``tests/``), the
smoke check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in it. The product path
(``context_attention_long_amd`` and its HIP library) never imports it, and it
never imports the product path: the two share no code, no headers, no helper,
no table and no constant generator. Only the seeded input generators in
``synth`` feed both sides, and those hold none of the method's arithmetic.

Each function states the passage of the source pages it writes out:

* "How GPUs Share a Long Context During LLM Inference" (vincentzed.com),
  called *Long Context* below: causal attention (1.1), zigzag (2.3),
  interleave (2.4), the partial-softmax problem (3.2), the LSE merge (3.3);
* the SGLang "Prefill context parallelism" documentation page, called
  *SGLang prefill CP*: "Zigzag strategy" and "Interleave strategy";
* the vLLM GLM-5.3 part-2 post on PCP/DCP/HiSparse, footnote 1 (FLOP count
  per key row and head);
* the vLLM "Decode Context Parallelism" post, section 4 (contiguous token
  chunks per GPU) and 5.3 (MLA: one latent vector shared by all heads);
* "DeepSeek-V4 Attention Inference Systems" notes, section 5 (the exact
  combine in max / sum / unnormalised-output form), sections 1 and 9.1
  (caches read through page tables of fixed-size logical blocks).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against page facts, closed forms, library routines or brute force; see each
module's header.
"""

from . import formats, plans, attention  # noqa: F401
