"""CPU fp64 attention oracle — test infrastructure only (see ``oracle.attention``).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It imports nothing from the product package and shares no code with it.
"""

from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
