"""CPU oracle for the hybrid GQA attention layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The product path (the HIP library and its Python binding) never does.
Every function is pinned by tests/test_oracle_pins.py; none is "parity unpinned".
"""
from .hattn_oracle import *  # noqa: F401,F403
from .hattn_oracle import __all__  # noqa: F401
