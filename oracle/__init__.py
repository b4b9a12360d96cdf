"""CPU oracle for MLA decode: TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check (__graft_entry__.smoke) and the benchmark's
CPU-baseline leg may import, call or execute anything in this directory.  The
GPU library must never route through it.  See mla_oracle.py for what it
computes and which passages it follows.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import __all__  # noqa: F401
from . import dsa_indexer  # noqa: F401,E402
from . import cache_append  # noqa: F401,E402
