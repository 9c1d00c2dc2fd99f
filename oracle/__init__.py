"""CPU oracle of the DiT denoising step -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product path (the HIP library and its binding)
never does.  See oracle/dit.py for the functions and the pages they follow.
"""
from . import dit  # noqa: F401
