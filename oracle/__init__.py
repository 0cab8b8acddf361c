"""CPU oracle for the lookahead decoding step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this package imports
nothing from the product path.  The only code both sides share is `synth`,
which draws seeded inputs and holds none of the method's arithmetic.

What it computes (plain, slow, fp64 numpy):

* `model`      -- a LLaMA-shaped decoder forward with an explicit boolean
                  visibility mask, plus bf16 rounding at the tensors the
                  bf16 contract stores in bf16.
* `lookahead`  -- plain greedy autoregressive decoding, and the lookahead
                  decoding loop step by step: 2D window, n-gram pool,
                  candidate selection, one forward pass under the lookahead
                  mask, greedy verification, window slide, pool insert.
* `attention`  -- one masked attention call with a materialised mask (the
                  attention kernel on its own).
* `scaling`    -- the closed forms of the pages' scaling law.

Citations name the page and its section / figure / equation:
  [LD]  "Break the Sequential Dependency of LLM Inference Using LOOKAHEAD
        DECODING" (the long-form analysis page, paper-graph-ui).
  [LDs] "Break the Sequential Dependency of LLM Inference Using Lookahead
        Decoding" (the short summary page, atlas.scime.ai).

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: a library LLaMA implementation (HF transformers, fp64), torch's
attention and bfloat16 conversion, closed forms, brute-force enumerations,
the pages' Fig. 1 / Fig. 2(b) examples, and the exactness invariant
(lookahead output == greedy autoregressive output).

Readings of points the pages leave open are listed at the top of each
module.
"""
