"""CPU oracle (test infrastructure only): see ``oracle.mla_oracle``.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path.
"""
from . import mla_oracle  # noqa: F401
