"""CPU oracle for lazy looped-Transformer inference (FlashLoop-style).

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float32 NumPy
statement of what the hot path computes.  Only the test-suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the library itself
never does, and this package imports nothing from the library (it shares no
code, tables or helpers with the HIP path).  Inputs come from the seeded
generator module, which holds no arithmetic of the method.

Sources followed (the pages the method is described on):

* FlashLoop abstract (arxivdaily.com, "FlashLoop: Fast and Memory-Efficient
  Looped Transformers via Lazy Updates", abstract): three observations --
  state changes concentrate on few tokens (token-sparse update), attention
  output differences are dominated by a sparse, stable subset of key columns
  (sparse attention), KV residuals between adjacent loops quantize well to
  low bit-widths (KV-residual quantization); each loop otherwise costs one
  more Transformer pass and one more KV set.
* FlashLoop walk-through (discosf.com): sandwich layout P + R x K + Q
  (section 3.1), loop embedding added to each loop's input, RoPE, residual
  state passing (section 3.2), inference flow (section 4.1), one KV cache per
  loop with shared projections (section 5.2), pre-LN (section 8).
* Looped Transformer tutorial (aiboss88.com): shared stack applied in a loop
  (step 1 pseudo-code), block-application counts (step 2, step 3, full
  example), per_loop / last_loop KV modes (step 4).

The pages give the three observations but no exact rules; the exact rules
used here are readings, each named where it is applied.  Parity status:
every function is pinned by the CPU tests (closed forms, brute force on tiny
inputs, reductions to library routines); whether these readings are the
FlashLoop authors' exact rules is unpinned, since the pages hold no worked
example, threshold or code.
"""
