"""fp64 CPU oracle for the DART hot path (test infrastructure only; see
``oracle/dart_oracle.py``).  The HIP library never imports this package."""
from .dart_oracle import *  # noqa: F401,F403
from .dart_oracle import __all__  # noqa: F401
