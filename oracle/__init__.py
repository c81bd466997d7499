"""CPU oracle for the packed ARCHead LM-head -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU implementation of what
the packed ARCHead head computes, written from the ARCHead paper
("Activation-Metric Residual Correction for LLM Output Heads", sections
3.1-3.3, equations 1-10).  It exists to check the HIP path.  Only the test
suite, the smoke entry point and the CPU-baseline leg of the benchmark may
import it; the product path (the C-ABI library and its Python binding) never
does, and there is no fallback from the product path into this code.

It shares no code with the HIP path: its own unpacking of the canonical byte
layout, its own fp16/bf16 decoding, its own quantiser and its own fp64
arithmetic.  Floating point is fp64 throughout.

Modules
-------
quant    symmetric b-bit quantiser with fp16 scales (eq 3 "Q_b", section 3.2;
         INT8 correction factors, text after eq 7)
layout   canonical byte layout: R4 nibble packing, fp16 / bf16 decoding,
         state-dict byte accounting (eq 10)
forward  dense fp64 W_hat (eq 6) and logits (eq 7), first-index argmax
packer   tiny-head construction (eqs 2-5): damped metric, core, SC4 residual,
         activation-metric correction, INT8 factors
naive    ctypes loader for naive.c, an independent triple-loop forward in C
select   top-k of the logits: larger value first, equal values by lower
         index (the argmax's tie rule widened to K candidates); top-k
         sampling at a temperature from a given uniform number
softmax  log-normaliser lse = log sum_v exp(logits) and cross-entropy
         lse - logit[target] of the logits (abstract and section 1: the
         logits feed the softmax; the head is judged by cross-entropy and
         perplexity)

Parity pins (what each function is checked against, in tests/):
  quant   -- closed-form bounds |x - s q| <= s/2, ranges, idempotence, and
             hand-worked examples in tests/golden/quant_examples.txt
  layout  -- round trip, hand-packed bytes in tests/golden/r4_nibbles.txt,
             eq 10 byte counts against the paper's 1187 MiB BF16 Qwen head
  forward -- the independent C triple loop, one-hot closed forms, special
             cases reducing to plain integer matrix products, a hand-worked
             example in tests/golden/forward_example.txt
  select  -- K = 1 against the pinned first-index argmax, Python-sort brute
             force on small rows with many ties, hand-built ties with +-0;
             sampling: K = 1, equal values, the two-way closed form, tau -> 0
  softmax -- closed forms (equal logits: ln V; V = 1; two-way softplus),
             shift invariance, softmax sums to one, math.fsum brute force on
             tiny rows, scipy's logsumexp at overflow-prone magnitudes
  packer  -- correction: Eckart-Young-Mirsky tail energy, brute force over
             random and grid rank-r candidates, the eigenvector route, the
             p = 1/2 identity with eq 1, the isotropic (C = I) reduction;
             core and SC4 residual, from W and the stored fields alone: the
             best rank-k approximation and tail energy by the eigenvectors of
             W^T W, sqrt(sigma_i) in each core column / row within the norm
             of the half-steps, residual scales fp16(absmax / 7) and codes
             within half a step of W minus the unquantised best rank-k
             product; planted mistakes (wrong triplets, sigma on one side,
             residual of the quantised core) each fail one of these
"""
