"""CPU oracle for the persistent decode megakernel -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package. The product
path (the HIP library and its Python binding) never touches it and shares no
code with it; the two meet only in the seeded input generator (``workload``),
which holds none of the method's arithmetic.

Contents
--------
``bf16``     bfloat16 encode (round to nearest, ties to even) / decode.
``decoder``  the plain pre-norm Llama-style decoder, one token per call, in
             float64 (bf16 only where the problem stores it: weights and the
             KV cache); no blocking, fusion or reordering.
``graph``    the fine-grained task graph written from its specification
             (tasks, events with thresholds, round-robin placement, canonical
             bytes), a replay of it in random topological orders, and a static
             race check.

Sources (the pages on compiling LLM decoding into one persistent kernel):
* Mirage Persistent Kernel blog translation (zejuncao.github.io, "MPK compiler"
  and "MPK runtime" sections, Figures 2 and 3): task/event semantics.
* MPK code walk-through (zizhi168.cn, section 3.3.1 "build_mirage_graph"):
  operator order and wiring of one decode step.
* Hazy Research megakernel news summary (sfrk.com.cn): the fused instruction
  list (RMSNorm+QKV+RoPE, attention matmul+reduction, O-proj+residual,
  RMSNorm+gate/SiLU+up, down+residual, final RMSNorm+LM head).

Parity pins for every function live in ``tests/oracle``. Nothing here is
"parity unpinned" except the greedy token ids / logits at random
initialisation themselves, which none of these sources prints (they are fixed only
through the invariants the tests check).
"""
