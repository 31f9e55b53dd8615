"""Reference oracle for the paged-KV GQA decode step (TEST INFRASTRUCTURE ONLY).

A plain, slow CPU implementation in numpy float64 of everything the HIP path
computes. It exists to check the GPU library and nothing else: only the test
suite, the smoke entry point and the benchmark's CPU-baseline leg may import
it. The product path never calls into this package, and this package imports
nothing from the product (no shared kernels, helpers, tables or constants).

Pages followed (cited by title and section in every function):

* mini-infer README -- "Project overview" (paged KV cache = BlockTable plus a
  free-block pool) and the four "decode_batch key steps" (gather through the
  block table, batched forward, write_decode_kv).
* On-device LLM inference course project (NJU) -- section 2.1, the list of
  components to implement: RMSNorm, RoPE, QKV projection with grouped-query
  attention (sdpa with enable_gqa, or repeat_interleave of the KV heads),
  SwiGLU MLP, decoder-layer assembly with residuals and two norms, KV-cache
  append.
* nxmr.cn inference-techniques article -- section 2.1 (page-table
  allocation, ceil(seq_len / PAGE_SIZE) pages), section 4.1 (attention scores
  in FP32), section 5.1 (numerically stable softmax: row max, exp, row sum).
* vLLM-based inference-framework project report (gitlink.org.cn) -- the
  "FP8 KV Cache quantisation" exploration (an 8-bit KV cache to cut the bytes
  moved); nxmr.cn article section 2.2 (per-head quantisation scales).
* MegEngine/InferLLM article (lnwmold.com) -- section 4.2 "problem two"
  (KV-cache size formula and its ~1 GB worked example), section 3.4
  (preallocated contiguous per-layer K/V cache).

Modules:
  bf16       bf16 <-> float64 codec (definition of round-to-nearest-even)
  fp8        E4M3 codec, per-head static-scale quantise / dequantise
  paged      block counts, slot mapping, free-block stack, size formula
  rope       rotary position embedding, half-split pairing
  attention  write_decode_kv, gather, paged GQA decode attention (bf16 and
             8-bit caches), the split-K partial statistics and their merge,
             prefill (packed prompt write, causal attention)
  layer      RMSNorm, SiLU, SwiGLU, full decoder-layer decode step
  sched      continuous-batching step planner with the KV brakes and swap

Every function is pinned by the ``-m "not gpu"`` tests against closed forms,
invariants, brute force or independent library routines. Any function without
such a pin says "parity unpinned" in its docstring.
"""
