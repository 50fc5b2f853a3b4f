"""CPU oracle for block-scaled low-precision GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``block_scaled_precision_bsgemm_amd`` and its HIP library) never
imports, links or calls it, and shares no code with it.

What it computes, in plain slow code, decoding every code exactly to float64:

* ``formats``  -- the element and scale formats (E2M1, E4M3, E8M0, BF16):
  exact decoders and round-to-nearest-even, saturating encoders.
* ``quantize`` -- the NVFP4, MXFP8 and MXFP4 quantizers (vectorised numpy,
  FP32 arithmetic emulated with numpy float32).
* ``scalar``   -- a second, independent scalar quantizer in pure Python with
  ``fractions.Fraction`` and its own FP32 rounding, used only to cross-check
  ``quantize``.
* ``gemm``     -- the block-scaled GEMM references (NVFP4 x NVFP4, MXFP8 x MXFP8,
  MXFP4 x MXFP4, grouped NVFP4 x BF16, NVFP4-weight x BF16-activation), the
  magnitude sum T[m,n] = sum_k |a_k b_k| and the per-element acceptance test.

Sources.  The pages this library follows name the formats but define none of
their arithmetic:

* "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera Rubin NVL72",
  section "Building the GEMM": block-scaled NVFP4 and FP8 E4M3 GEMMs at 16k
  square, B shared by two M-stacked output tiles.
* "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve Tensor-Memory
  Failures", sections "The missing case was defined by shape, layout, and
  execution mode together" and "Ragged mode added routing rather than a plain
  matrix": NVFP4 (nvfp4_e2m1) activations x dense BF16 operand, ragged routing,
  BF16 output.
* "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic" (bitsandbytes
  PR #2030), section "Methodology": fused 4-bit-weight GEMM with BF16
  activations, checked against an FP32 dequantise-then-linear reference.

The bit layouts follow the OCP Microscaling Formats (MX) v1.0 specification
(E2M1, E4M3 "FN", E8M0) and NVIDIA's published NVFP4 description (E2M1 values,
one E4M3 scale per 16 elements, one FP32 per-tensor scale).  The quantizer
recipes (tensor scale = absmax / (6 * 448), block scale = (block absmax / 6) /
tensor scale, MXFP8 block exponent = ceil(log2(block absmax / 448)), MXFP4
block exponent = ceil(log2(block absmax / 6))) are the
problem statement of this library; every reading taken where that statement is
silent is listed in the docstring that takes it.
"""

from . import formats, quantize, scalar, gemm  # noqa: F401
