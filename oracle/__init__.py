"""CPU oracle for the Llama 4 mixture-of-experts feed-forward block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or
runs this package; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP path: the two meet only
at the seeded input generator (package `synth`), which holds no arithmetic of
the block.

Contents
  numerics  bf16 and OCP e4m3fn rounding written from the format definitions
  block     the block itself in fp64 (router, top-1, sigmoid gate on the
            input, routed + shared SwiGLU experts, combine) with the
            rounding points of the reduced-precision variants emulated;
            the optional RMSNorm in front, k experts per token, dense
            layers (no routed experts), and int8 / int4 / e4m3 weight codes
            dequantised with their column scales
  brute     pure-Python loops that evaluate every expert densely, then select
  arith     the pages' parameter / FLOP / KV-cache arithmetic

What the block computes is taken from: the KerasFormers "Llama 4" page,
section "What is unusual about the block" (top-1 of 16 / 128 experts, a
routed expert's input multiplied by the sigmoid of its logit, a shared MLP
alongside the experts); the
superteams.ai glossary "Llama 4", section "Mixture of Experts: Why Total and
Active Parameters Diverge" (one logit per expert, argmax, the shared
expert's output plus the routed expert's output, the other experts idle);
and the "Llama 4 Maverick" page of llm-architectures-explained, table "Every
architecture field" (experts are gated MLPs of width intermediate_size, one
shared expert of the same width).

Parity pins: every function is pinned by tests under tests/ that run
without a GPU (brute force, closed forms, special cases reducing to library
routines, invariants).  "Parity unpinned": none of the pages prints a worked
numeric example of the block's output, so output numerics at full size are
pinned only through brute force at tiny size.
"""
from . import numerics, block, brute, arith  # noqa: F401
