"""CPU oracle for dynamic top-K sparse decode attention — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The HIP library never
calls it and shares no code with it.

``reference`` is the plain, slow, fp64 numpy implementation; ``brute`` is an
independent pure-Python (no numpy) re-derivation for tiny shapes.

Parity status of each function is recorded in its docstring; none is
"parity unpinned" except the aggregate statistics of the ReTopK run on
synthetic AR(1) queries (reuse ratio, mean candidate count), which the pages
only report for real model activations and which are therefore reported, not
checked.
"""

from . import reference  # noqa: F401
