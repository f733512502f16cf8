"""Float64 CPU oracle of the MoE-layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library's product path never
does.  It shares no code with the HIP library (no kernels, headers, helpers or
tables) and imports nothing from it.

* ``moe_oracle`` -- NumPy float64 implementation of the plain definitions.
* ``brute``      -- pure-Python (stdlib only) per-token brute force for tiny
                    inputs, used to cross-check ``moe_oracle``.
"""
from . import moe_oracle, brute  # noqa: F401
