"""CPU oracle for the SVDQuant W4A4 + low-rank linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or call anything in this package.  The library (``bit_diffusion_model_amd``) never
imports it and shares no code with it.

Everything here is plain numpy in fp64 (floating point) and exact integers, written
step by step from the pages that describe the method:

* the SVDQuant review at jeonghoonpark.com ("SVDQuant", sections 3 "Quantization
  Preliminary", 4.2 "SVDQuant: absorbing outliers via low-rank branch" and 4.3
  "Nunchaku"),
* the SVDQuant abstract at chatpaper.ai (LoRA support without re-quantization),
* the ch3chohch3.github.io post "从 Smooth Quant 到 SVD Quant" (the smoothing
  equation and smoothing-factor formula, the SVD truncation and the static/dynamic
  quantization split).

Where the pages leave a step open, the reading taken is stated in the docstring of
the function that implements it.

Pin status: every function is pinned by the ``-m "not gpu"`` tests against closed
forms, exhaustive sweeps, independent exact (``fractions``) evaluations, library
reductions or brute force, except the absolute output values of the full layer on the
named workloads: the pages print no worked example for them, so those are pinned only
through their pinned parts (quantizers, group sums, SVD identities) and brute force on
tiny shapes.
"""

from . import numerics, quant, pack, forward, weight_only  # noqa: F401
