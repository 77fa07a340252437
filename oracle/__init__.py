"""Float64 CPU oracle of the CSA hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It shares no code with the HIP path (libcsa and its binding) and
imports nothing from it; the two meet only in the seeded inputs of ``datagen``.
"""
from . import csa, pipeline  # noqa: F401
