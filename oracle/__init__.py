"""CPU oracle for the chunked TTT-KVB fast-weight layer -- TEST INFRASTRUCTURE.

This package is a plain, slow, obviously correct NumPy implementation of what
the GPU library computes. It exists only to check the GPU library. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the library and its Python binding never do, and nothing here imports
them. It shares no code with the HIP path: no kernels, headers, helpers,
tables or constants.

Arithmetic is float64 by default (``dtype`` arguments allow float32 for
timing). Every step follows the pages in their order and notation:

* ``oracle.lact``     -- the LaCT layer: SwiGLU fast weight, gradient of the
  eta-weighted negative inner-product loss, momentum, Newton-Schulz-5,
  input-dim renormalisation, apply/update order.
* ``oracle.linattn``  -- the last-layer-only linear-attention form
  ``O_c = phi(Q_c) S_c`` with ``S_c = W1 + sum of earlier chunk aggregates``.
* ``oracle.inplace``  -- the In-Place TTT down-projection update.

Readings of passages that the pages leave open are listed with each function.
"""
from . import lact, linattn, inplace  # noqa: F401
