"""CPU reference ("oracle") for pipelined self-speculative decoding of looped Transformers.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this package:
only the tests, the graft smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the GPU path (`looped_transformer_self_amd`); both are fed the
same seeded inputs from `synth`.

What it computes, and where the pages define it (LoopSpec page, liuzhao09.github.io,
"LoopSpec: Pipelined Self-Speculative Decoding for Looped Transformers"):

* `model`    - the looped model P -> B^r -> C of section 2.1, eq. 1, with per-depth KV
               caches (depth-indexed, never mixed across loop depths: section 2.1, Fig. 2,
               and section 2.4).  Plain NumPy, float64 arithmetic; tensors that the model
               stores in a reduced precision (weights, GEMM inputs, KV cache: BF16 per
               section 3.1) are rounded at exactly those points.
* `readout`  - C's temperature, optional top-p truncation and normalisation (section 2.1).
* `sampler`  - residual operator (eq. 2), single-candidate rejection (eq. 3-4), residual
               second proposal and gate (eq. 5-6), cascade verification (section 2.3),
               written in integer fixed point so decisions are bit-reproducible.
* `philox`   - Philox4x32-10 counter-based generator (Salmon et al., SC'11) for the
               position-keyed uniforms both sides consume.
* `decode`   - plain full-depth autoregressive decoding (the target the method must
               match) and a serial speculative decoder making the same decisions the
               pipelined decoder makes, one position at a time.
* `copyprop` - copy-suffix candidate proposer with shallow screening (CopyLoop page,
               kongchang.com, "CopyLoop"), one reading of a rule the page leaves open.

Parity unpinned: the copy-suffix candidate rule and screening threshold (they change
speed only, never the committed distribution).
"""
