"""fp64 CPU oracle for KDA prefill.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg may import anything here; the GPU library and its Python
binding never do, and the two share no code.

* ``kda_oracle.c`` / :func:`prefill` -- the plain token-by-token recurrence in
  double precision (the definition of the result).
* ``kda_oracle.c`` / :func:`backward` -- its reverse-mode gradients, token by
  token in double precision.
* :mod:`oracle.reference` -- NumPy forms used to pin the oracle: the explicit
  K x K matrix product form, and the 16-token chunked form with its
  per-chunk intermediates.
"""
from .kda_oracle import backward, build, prefill, library_path, max_threads  # noqa: F401
