"""CPU oracle of the product-key memory lookup (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .pkm_oracle import *  # noqa: F401,F403
