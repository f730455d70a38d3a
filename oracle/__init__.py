"""CPU oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy/fp64 implementations of what the hot path
computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package; the product path (the HIP library
and its Python binding) never does, and this package imports nothing from it.

Sources, the Kshipra blog series:
  [K2] "KV-Caching, Batching, and Memory Complications: Scaling Kshipra on CPU"
       (blog/kshipra-2), section 1 "KV-Caching" (decode appends the new K/V
       and attends over the cache including itself) and section 2 "Static
       Batching & the Left-Padding Position Bug" (the first real token has
       absolute position 0; a decode token sits at position length - 1).
  [K3] part 3 of the series (blog/kshipra-3):
       section 1 "Block-Arena KV Cache": arena of fixed-size blocks, LIFO
         free list, GQA-aware sizing                      -> pool, arena
       section 3 "Radix-Tree Prefix Cache": shared blocks kept alive by
         reference counts; a block that diverges is copied before it is
         written; least-recently-used leaf eviction that re-scans the tree
                                                          -> pool, radix
       section 5 "Continuous Batching and Admission Control": admission
         rule; preemption by swapping blocks out         -> pool, arena
       section 2 "INT4 Quantization and the Scale Bug": group quantization
         with one FP16 scale used to encode and decode   -> quant
       section 4 "Chunked Prefill": online softmax over blocks read in place,
         RoPE at absolute positions P onward, causal mask over the chunk,
         result identical to dense masked attention       -> rope, attention

Modules:
  rope       closed-form rotary embedding, cos/sin tables from libm in fp64
  pool       LIFO free list + reference counts + copy-on-write + admission
  radix      radix-tree prefix cache with re-scanning LRU eviction
  arena      block-arena writes/gathers, materialised (fp16/fp32 or
             group-quantized) or symbolic
  quant      group quantization codec (INT8/INT4 codes, FP16 scale)
  attention  dense gather, masked score matrix, two-pass softmax in fp64
  script     runs a workload's pool script and step on the above

Parity pins for every function live in tests/test_oracle_*.py.
"""
from . import rope, pool, arena, attention, quant, radix, script  # noqa: F401
