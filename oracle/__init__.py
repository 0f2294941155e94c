"""CPU oracle for the AWQ W4A16 hot path (test infrastructure only).

Importable only from the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.
"""
from .awq_oracle import *  # noqa: F401,F403
from . import awq_oracle  # noqa: F401
