"""CPU oracle for the FlashHead output head -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy restatement of what the FlashHead paper
("FlashHead: Efficient Drop-In Replacement for the Classification Head in
Language Model Inference", Section 3 and Appendix D.1) computes.  It shares no
code with the HIP library under ``clustered_retrieval_lm_amd/`` and never
imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path must not.

Modules
  philox    Philox4x32-10 counter-based uniforms and Gumbel noise
  codecs    bf16 round-to-nearest-even and the int4 group-128 format
  kmeans    balanced spherical k-means (offline clustering)
  head      dense head, tile packing, FlashHead forward (greedy and sampling)
  marginal  closed-form two-stage sampling marginal and the Monte-Carlo
            estimator of Appendix D.1

Pins (what each function is checked against, in tests/test_oracle_*.py):
  philox    rocRAND's Philox4x32-10 engine (a separate implementation of the
            same published generator); uniformity chi-square
  codecs    torch's CPU float32->bfloat16 conversion; int4 round-trip bound
  kmeans    balanced-cluster invariants, exact latent-partition recovery on
            well separated data, brute-force repair order on tiny inputs;
            large-config clusterings are PARITY UNPINNED beyond invariants
  head      exact integer arithmetic through pure-Python loops, dense head at
            p = c, brute-force top-p
  marginal  p = 1 product form, p = c full softmax, chi-square of the sampler
            against the enumeration, Appendix D.1 normalisation
"""
