"""Plain fp64 CPU oracle for the TQ4_1S ("Config-I") dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, calls or
links it, and it shares no code, table or constant generator with that path.
"""

from .fp8_oracle import *  # noqa: F401,F403
from .fp8_oracle import __all__ as _fp8_all
from .tq4_oracle import *  # noqa: F401,F403
from .tq4_oracle import __all__ as _tq4_all

__all__ = list(_tq4_all) + list(_fp8_all)
