"""CPU oracle for the VC-Attention forward pass (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP library never does, and this package imports
nothing from it.
"""
from .vc_oracle import *  # noqa: F401,F403
from . import vc_oracle  # noqa: F401
