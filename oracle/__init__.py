"""CPU oracle (test infrastructure only): see ``oracle.oracle``.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  It shares no code with the HIP path."""
from .oracle import *  # noqa: F401,F403
from .oracle import __all__  # noqa: F401
