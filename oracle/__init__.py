"""CPU oracle for low-rank KV-cache decode attention and the append/quantise path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the HIP library.

What it follows
---------------
* TraceKV ("TraceKV: Policy-Preserving Low-Rank KV Cache Compression for
  Reasoning Vision-Language Models", abstract): the cache stores
  low-dimensional latents of the KV states, optionally quantised, and
  attention runs from those latents.
* ai4snews page on TraceKV, Synopsis: 70% rank ratio combined with 4-bit
  quantisation; Perspective: decode latency at batch 16, 4K-32K context.
* iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental
  SVD", English abstract): an exact recent window is kept while older tokens
  are folded into the bounded-rank latent history.

Modules
-------
``attention``  D1 reconstruct-then-attend, D2 latent-domain, D3 pure-Python brute force.
``quant``      int4 groups-of-32 min-max quantiser, nibble packing, exact dequantiser.
``append``     the append state machine: exact window ring, eviction, projection, storage.
``rebase``     historical-coordinate sync after a basis update (least-squares coordinates).
``basis_update`` block-incremental basis update (Brand's incremental SVD of [diag(sigma) B ; Y])
               and the sync weights W = B' B^T it hands to the coordinate sync.
``sensvd``     sensitivity-weighted SVD basis construction (top-r right singular vectors).
``rankalloc``  global rank allocation: greedy marginal energy gain under a total budget.
``prefill``    chunked prefill attention: a chunk's queries over the latent history, the exact
               window and the chunk itself (causal); P1 reconstruct, P2 latent, P3 brute force.

Every function works in float64 unless the step it models fixes a narrower
precision (the quantiser's float32/float16 steps, storage rounding).

Parity status: every function here is pinned by tests under ``tests/``
(closed forms, a library routine, invariants and brute force); see each
module's header for the pins.
"""
