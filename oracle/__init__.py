"""CPU oracle for the FastMTP verify step through the MoE decoder.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP library
and its Python binding never do, and this package imports nothing from them.

See ``oracle.moe`` for the definitions and their sources.
"""
from .moe import *  # noqa: F401,F403
from .moe import __all__  # noqa: F401
