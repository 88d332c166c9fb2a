"""CPU oracle of the VSA operator (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP path never does.
"""
from . import vsa_oracle  # noqa: F401
