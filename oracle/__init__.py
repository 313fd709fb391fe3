"""CPU oracle for the ternary linear layer (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .twl_oracle import *  # noqa: F401,F403
