"""CPU oracle for the Fast-BLT local byte decoder step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only the test-suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP path;
the only thing both sides consume is the seeded input generator ``bltgen``.

It is a plain, slow, float64 NumPy restatement of what the method computes,
written from the Fast-BLT descriptions:

  * pytorch.kr Fast-BLT summary ("Fast Byte Latent Transformer (Fast-BLT)
    연구 소개"), sections on the BLT architecture, BLT-D inference, the BLT-D
    attention masks, the unmasking strategies, BLT-S/BLT-DV verification and
    the efficiency metrics;
  * wangzhan123.com Fast-BLT article, section six (how efficiency is
    measured), which spells out the bandwidth formula in words.

Modules:
  model    -- decoder forward with explicit attention masks (no cache)
  cache    -- the same forward over a clean-prefix KV cache
  decide   -- softmax/argmax/confidence, unmask-and-commit, verify-accept
  patcher  -- stand-in patch segmentation rule and cross-attention targets
  loops    -- greedy BLT, BLT-D, BLT-S and BLT-DV decode loops with counters
  proxy    -- the pages' parameter-load bandwidth proxy

Every function whose result is not pinned by a test against the pages or the
mathematics says "parity unpinned" in its docstring; at present none does.
"""
