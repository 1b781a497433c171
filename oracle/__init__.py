"""Plain fp64 CPU oracle for the HSQ decode step and the TurboQuant codec.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, tables or
constants with the HIP library; both sides only consume the same seeded inputs.

Every function states the passage it follows.  Sources (web pages):

* "Tamarin (HSQ) - reversible hierarchical KV-cache compression" technical
  summary, in Korean and in Dutch (same content): section 2 "Methodology"
  with its parts "Three-tier architecture", "Decode process" and "Key
  technical components".
* "Ablation, Statistical Inference, and Validation for KV-Cache Compression"
  technical summary: "Experimental setup" (TurboQuant: random Walsh-Hadamard
  transform followed by a data-oblivious Beta Lloyd-Max codebook) and
  "Key contributions" section 2 (Jensen amplification of key-path errors).

Modules:
  codebook   Beta Lloyd-Max codebook for the coordinate marginal of a uniformly
             random unit vector.
  codec      random-sign Walsh-Hadamard rotation, norm scaling, scalar
             quantisation, 4-bit / 3-bit packing, dequantisation.
  tiers      L1 / L2 / L3 tier plan and build.
  cache      decode-time tier maintenance: append a token, evict from the
             recent window, seal N pending tokens into a group.
  decode     router scores, top-beta, union-set softmax attention, dense
             attention.
  qjl        TQ-QKV: 1-bit QJL sketch of the key residual and the corrected
             logits.
  rope       pre-RoPE archive: dequantise, then rotate to the token's
             position.
"""
