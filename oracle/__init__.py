"""CPU oracle for the dropless MoE layer forward -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct statement of what the MoE
layer forward computes, written in numpy float64 from the pages that define the
method:

* "Scalable Training of Mixture-of-Experts Models with Megatron Core" (summary
  page), section "Method", first paragraph: the layer is a router (a learned
  linear projection, optionally evaluated in FP32, then softmax or sigmoid
  scores, then top-k selection), a dispatcher that permutes tokens so that all
  tokens routed to one expert are contiguous, experts that run together as one
  grouped GEMM, and a combine step; an optional shared expert runs on every
  token.
* Same page, "Method", second paragraph, and "Key claims" (the [§5] item): the
  router stays in higher precision while expert GEMMs may run in FP8.
* The same paper's index page, abstract: dropless MoE with Grouped GEMM,
  fusions and sync-free execution.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding under ``mixture_experts_layer_fp32_amd/``) never imports it and
shares no code with it; the only thing both sides consume is the seeded input
generator in ``moe_inputs/``, which holds none of the method's arithmetic.

Modules
-------
``oracle.e4m3``  OCP FP8 E4M3 ("e4m3fn") codec and 1x128 / 128x128 block
                 quantisation, from the format definition.
``oracle.moe``   the stages Route -> Dispatch -> Compute -> Combine, each as
                 its plain definition, plus a pure-Python brute-force layer.
"""

from . import e4m3, moe  # noqa: F401
