"""Float64 CPU oracle for GVA decode -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .gva_oracle import *  # noqa: F401,F403
from .gva_oracle import __all__  # noqa: F401
