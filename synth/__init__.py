"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws random numbers and lays them out; it holds none of the
quantization or GEMM arithmetic.  All tensors are bf16, generated from a
seeded torch Generator:

* ``randn_bf16``: N(0, 1) drawn in float32, rounded to bf16 (activations X,
  gradients dY; the pages build A with ``randn``).
* ``linear_weight_bf16``: U(-1/sqrt(K), 1/sqrt(K)), the distribution that
  ``nn.Linear(K, N)`` initialises its weight with (kaiming-uniform with
  a = sqrt(5)), rounded to bf16.  The repro the pages describe uses a
  deterministic ``nn.Linear`` weight for B.

Host generation (``device="cpu"``) is used for everything the oracle checks
element by element; large bench-sized inputs may be generated on the GPU
with the same recipe (``device="cuda"``) and sampled back to the host.
"""

from .inputs import (randn_bf16, linear_weight_bf16, bf16_bits, to_device,  # noqa: F401
                     tensor_seed)
