"""Plain, slow CPU oracle of the DP-SGD per-sample clipping hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
of the entry module and the CPU-baseline leg of the benchmark may import or
run anything in this package. It shares no code with the HIP library or its
Python binding; neither side imports the other.

Contents:
  definitions  fp64 definitions: per-example gradients (materialised), their
               norms, the layerwise path rule, clip factors, the clipped sum,
               the noised mean and the adaptive threshold.
  noise        the counter-based Philox4x32-10 + Box-Muller normal stream,
               evaluated with numpy fp32 operations in a fixed order.
  drivers      whole layer-set steps built from the two modules above.

Parity status: every function is pinned by a CPU test against something other
than itself (brute-force autograd, closed forms, identities, invariants,
published Philox known-answer vectors, sample statistics). The Philox counter
layout and the Box-Muller operation sequence are a specification chosen here
(the pages name no generator); they are pinned only by the known-answer
vectors, the statistics tests and the accuracy checks of ln/sin/cos.
"""
