"""fp64 CPU oracle of the LISA layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library and its Python binding never do.
"""
from .lisa_oracle import *  # noqa: F401,F403
