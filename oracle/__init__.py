"""fp64 CPU oracle of the Lens MM-DiT denoiser step.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The HIP library never uses it, and it shares no code with the HIP library.
"""
from .lens_oracle import *  # noqa: F401,F403
