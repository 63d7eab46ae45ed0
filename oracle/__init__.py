"""Test infrastructure: a plain, slow fp64 CPU oracle of the MuonClip optimizer step.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package.  The product path
(``muonclip_muon_amd`` and its HIP library) never does, and this package never
imports the product: the two share no code.
"""

from .muonclip_ref import *  # noqa: F401,F403
from .rounding import *  # noqa: F401,F403
