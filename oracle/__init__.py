"""CPU oracle for the Llama-style decode step (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never calls it.
"""
from .llama_decode import *  # noqa: F401,F403
