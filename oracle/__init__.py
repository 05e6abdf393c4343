"""CPU oracle for paged decode attention.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never does: it shares no code, header,
table or helper with this package, and the binding fails loudly when the HIP
library is missing rather than falling back to anything here.

Every function is a plain, slow, obviously correct statement in float64 of
what the pages define; see ``pagedkv_oracle`` for the function-by-function
citations.  Parity status of each function is recorded in that module's
header.
"""
from .pagedkv_oracle import *  # noqa: F401,F403
from .pagedkv_oracle import __all__  # noqa: F401
