"""CPU oracle for one NanoFlow decoder-layer iteration — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 NumPy code that states what the layer computes, so
that the GPU library can be checked against it. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import anything from this package; the product path never
does, and this package imports nothing from the product.

Contents
--------
``layer``    the layer itself (token layout, paged-KV slots, RMSNorm, projections, rotary
             embedding, paged causal GQA attention, SwiGLU FFN, KV write) and a FLOP counter.
``schedule`` dependency rule between nano-operations, a list-schedule simulator and a
             brute-force two-stage pipeline search over small discrete spaces.
``costmodel`` the pages' analytical cost model (memory, compute and network time, the
             classification ratio, optimal throughput, roofline and KV sizing).

Sources: "NanoFlow: Towards Optimal Large Language Model Serving Throughput" (the
paper-graph-ui summary page: "The Cost Model and the Compute-Bound Classification", "The
Intra-Device Parallelism Mechanism", "Auto-Search Stage I", "Auto-Search Stage II") and the
NanoFlow OSDI'25 slides (8B pipeline design, Stage 1/Stage 2 constraint slides, batch
formation); paged KV semantics follow "LLM Inference Performance" (PagedAttention section)
and "Inside nano-vLLM" (paged KV, prefill batching sections).

Parity status per function is stated in each module's header.
"""
