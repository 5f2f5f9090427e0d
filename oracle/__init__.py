"""CPU oracle for the TurboQuant KV-cache decode path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product path
(the HIP library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product path.

Everything here is plain NumPy in float64, written so that each step can be
checked by eye against the pages it cites:

* "TurboQuant Performance Benefits: Memory Reduction and Speed Optimization
  in MLX-VLM" (mlx-vlm performance page),
* "How to Use TurboQuant with the MLX-VLM Python API: A Complete Guide"
  (mlx-vlm API page),
* the "mlx-turboquant" README (mlx-lm adapter page).

Parity pins: every function below is pinned by a CPU test in tests/
(closed forms, library routines, brute force on tiny inputs, statistics).
No function here is "parity unpinned".
"""

from .turboquant import *  # noqa: F401,F403
from .affine import *  # noqa: F401,F403
