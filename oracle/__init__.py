"""CPU oracle for pooled block-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and the two share no code.
"""
from .oracle import *  # noqa: F401,F403
