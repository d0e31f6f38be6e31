"""CPU oracle for the QSA decode step -- test infrastructure only.

Only the tests, the graft smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does.
"""
from . import qsa_oracle  # noqa: F401
