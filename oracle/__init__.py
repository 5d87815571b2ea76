"""Plain CPU oracle for the sparse MoE layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports or calls it.
"""

from .moe_oracle import *  # noqa: F401,F403
