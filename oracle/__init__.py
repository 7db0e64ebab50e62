"""CPU oracle for the ConvRot INT4 weight-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import,
call or link anything here.  The product library (``include/w4.h`` and the
``int4_weight_quantized_block_amd`` package) never touches this package, and
this package never imports the product.  The two share no code: the only module
both are fed from is ``synth`` (random inputs, none of the method's arithmetic).

The oracle is deliberately plain and slow: fp64 for every floating-point step,
an explicit g x g Hadamard matrix multiply per group (no butterflies), NumPy's
``rint`` for round-half-to-even, bit operations for nibble packing, and a plain
C triple loop with 64-bit accumulation for the integer GEMM.  See
``oracle/ref.py`` for each step and the passage it follows.

Pins (``tests/test_oracle_*.py``, run with ``-m "not gpu"``) tie it to facts
that do not come from the oracle itself: the Hadamard closed form against the
Sylvester recursion, orthogonality, exact rational recomputation on tiny
inputs, brute-force arg-min quantization, all 256 byte values for the nibble
codec, a Python-int GEMM, and torch's own bf16 cast.  One function carries no
such pin and is marked "parity unpinned" in its docstring.
"""
from .ref import *  # noqa: F401,F403
from .ref import __all__  # noqa: F401
