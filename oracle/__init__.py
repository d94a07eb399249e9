"""CPU oracle (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package.  It shares no code with the HIP path.
"""
from . import dit  # noqa: F401
