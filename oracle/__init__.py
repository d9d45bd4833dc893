"""fp64 CPU oracle for paged decode attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this package
imports nothing from the product path: the two share no kernels, headers, helpers,
tables or constants.  Only the seeded input generators in ``synth`` feed both.

What the oracle follows (pages cited by title and section):

* "PagedAttention: Optimizing KV Cache in vLLM" (grasp.study lesson), §3 "Making it
  Work: The PagedAttention Kernel": the block-aware kernel walks a request's blocks
  in logical order with a running softmax and reaches the same result as attention
  over contiguous K/V; paging changes the memory layout, not the mathematics.  The
  oracle is therefore that definition written out — softmax attention over each
  sequence's contiguous K/V in float64 (``attention``).
* Same lesson, §4 "Advanced Benefit: Zero-Cost Sharing with Copy-on-Write", and
  "What is PagedAttention?" (qubittool glossary), "How It Works": block tables,
  on-demand allocation, reference counts and copy-on-write of a shared block before
  a write (``allocator``: a plain dict model).
* The pool's byte layout, the fp8 e4m3fn format and the slot convention are this
  project's ABI (declared in ``include/pagedkv.h``) and the OCP 8-bit float format;
  ``pool`` and ``codecs`` implement them from those definitions.

Every function here is pinned by the ``-m "not gpu"`` tests against brute force,
closed forms, library routines or the format definitions; see each module.
"""
