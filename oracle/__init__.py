"""CPU oracle for the INSTANT low-rank backward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``. The product library
(``rank_compressed_backprop_amd``) never imports it and shares no code with it.
"""
from .instant_oracle import *  # noqa: F401,F403
from .instant_oracle import __all__  # noqa: F401
