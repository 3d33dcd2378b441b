"""CPU oracle for causal FP8/BF16 prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything in this package: only the test suite, the package-level
``smoke()`` check and the ``cpu_baseline`` leg of the benchmark use it.  It shares
no code with the HIP path (no kernels, headers, helpers, tables or constant
generators); both sides only consume the same seeded synthetic inputs.

Sources (the pages this follows; cited below by the short tags in brackets):

* [KG-en]  "Breaking the FP8 Attention Bottleneck on AMD MI355X: How Zyphra ZYFA
  Unleashes Performance" (kg.zhiyong.dev, English article).
* [MTP]    "Zyphra ZYFA: FP8 FlashAttention for AMD MI355X, Up to 1.76x Faster"
  (MarkTechPost reprint on news.qianmian.ai).
* [KG-zh]  the Chinese version of [KG-en] (kg.zhiyong.dev/insights), whose
  section on the technical solutions carries the full sentence that [KG-en]
  cuts off.

Modules:

* ``e4m3``        - OCP e4m3fn decode / round-to-nearest-even encode, bf16 RNE.
* ``attention64`` - the plain definition of causal softmax attention in fp64 on
  dequantised inputs (the target the method approximates).
* ``rotate``      - the Hadamard rotation of Q and K before their per-tensor FP8
  quantisation, and that quantisation.
* ``emulate``     - the FP8 method step by step (per-64-key-block power-of-2
  scaling, exact-exp or Lean-P probabilities rounded to e4m3, normalisation by
  the sum of the rounded probabilities), in fp64 except where the method rounds.
"""
