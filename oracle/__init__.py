"""Plain fp64 CPU oracle for the paged GQA attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or execute anything in this package; only
the tests, the smoke check of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the GPU path.
"""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
