"""CPU oracle of the low-bit MoE FFN layer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library never calls it
and shares no code with it; its inputs come from ``synth`` alone.

Pinning status (what each function is checked against, in tests that
need no GPU):

* unpack / decode_bf16 / decode_fp16: hand-written byte and bit-pattern
  fixtures (tests/golden) and a round trip through the generator's packer.
* router_logits: pure-Python sums on small inputs; a one-hot token gives
  the router row exactly; scaling x by 2^m scales the logits exactly; the
  prior adds per expert.
* route_topk: numpy's stable argsort and scipy's softmax; sum-to-one;
  k = E equals a full softmax; pure-Python brute force.
* permute: numpy bincount / cumsum / stable argsort; inverse identity.
* quant_rows_a8: hand-worked values (exact ties, zero rows) and a brute
  force that rounds an fp64 quotient to fp32 (innocuous double rounding).
* gateup / down / combine (A16 and A8): pure-Python per-token, per-expert
  loops; the E=1, k=1 case against a dense dequantize-then-matmul SwiGLU
  FFN; closed forms for one-nonzero-code layers; x = 0; scaling x by 2^m.

Parity unpinned (nothing on the pages fixes these; they are readings of
the layer definition and each test asserts them explicitly): the shared
expert's combine weight 1.0, the int2 scale rule (max|w|/1), the Zipf
prior reading, and rounding h to bf16 between the two A16 projections.
"""
from .moe_oracle import *  # noqa: F401,F403
