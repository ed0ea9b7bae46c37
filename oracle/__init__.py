"""CPU oracle for the QLoRA NF4 linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product (the HIP library and its
Python binding) never imports, links or executes it, and shares no code with it.
"""
from . import linear, nf4  # noqa: F401
